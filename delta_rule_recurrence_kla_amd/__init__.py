"""Python binding of libkla, the MI355X (gfx950) KLA forward hot path.

Argument marshalling only: tensors are checked for dtype/shape/device, their
device pointers and the current HIP stream are handed to the C ABI declared in
include/kla.h, and a non-OK status raises RuntimeError with kla_last_error().
Every step of the computation runs in the library's HIP kernels; there is no
fallback. PyTorch provides device memory and streams.

    out, S = chunk_fwd(q, k, v, log_alpha, eta, eps, init_state=None)
    out, S = chunk_fwd_psd(uq, uk, v, log_alpha, eta, eps)     # q, k = psi(u) formed in the kernels
    out = decode_step(q, k, v, log_alpha, eta, state, eps)     # state updated in place
    out = loglinear_decode_step(q, k, v, log_alpha, eta, lam, states, t, eps)  # Fenwick buckets
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "chunk_fwd_psd", "chunk_bwd", "decode_step", "loglinear_decode_step", "loglinear_fwd", "plan",
           "version", "last_error", "timing_enable", "timing_select", "timing_collect", "workspace_trim", "lib_path",
           "load", "KLAError", "PATHS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "lib", "libkla.so")
_lib = None

KLA_OK, KLA_ERR_INVALID_ARG, KLA_ERR_UNSUPPORTED, KLA_ERR_HIP, KLA_ERR_OOM = range(5)
PATHS = {"auto": 0, "sequential": 1, "scan": 2}
BETA_MODES = {"kaczmarz": 0, "direct": 1}
DTYPES = {"bf16": 0, "f32": 1}
_PATH_NAMES = {v: k for k, v in PATHS.items()}
_STATUS_NAMES = {0: "KLA_OK", 1: "KLA_ERR_INVALID_ARG", 2: "KLA_ERR_UNSUPPORTED", 3: "KLA_ERR_HIP", 4: "KLA_ERR_OOM"}


class KLAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class KernelTiming(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int), ("total_ms", ctypes.c_double)]


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libkla.so (built in tree by delta_rule_recurrence_kla_amd.build). Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"libkla.so is not built ({_LIB_PATH}); run "
                           "`python -m delta_rule_recurrence_kla_amd.build` first")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.kla_chunk_fwd.argtypes = [P, P, P, P, P, F, P, P, P, I, I, I, I, I, I, P]
    lib.kla_chunk_fwd_f32.argtypes = [P, P, P, P, P, F, P, P, P, I, I, I, I, I, I, P]
    lib.kla_chunk_fwd_ex.argtypes = [I, I, P, P, P, P, P, F, P, P, P, I, I, I, I, I, I, I, I, P]
    lib.kla_chunk_fwd_noalloc.argtypes = [I, I, P, P, P, P, P, F, P, P, P, I, I, I, I, I, I, I, I, P]
    lib.kla_chunk_fwd_psd.argtypes = [P, P, P, P, P, F, P, P, P, I, I, I, I, I, I, I, I, P]
    lib.kla_plan.argtypes = [I, I, I, I, I, I, I, I, I, I, ctypes.POINTER(I), ctypes.POINTER(I), ctypes.POINTER(S)]
    lib.kla_decode_step.argtypes = [P, P, P, P, P, F, P, P, I, I, I, I, P]
    lib.kla_decode_step_f32.argtypes = [P, P, P, P, P, F, P, P, I, I, I, I, P]
    lib.kla_decode_step_ex.argtypes = [I, I, P, P, P, P, P, F, P, P, I, I, I, I, P]
    lib.kla_loglinear_decode_step.argtypes = [I, I, P, P, P, P, P, P, F, P, P, I, I, I, I, I, I, P]
    lib.kla_loglinear_fwd.argtypes = [I, I, P, P, P, P, P, P, F, P, I, I, I, I, I, I, I, P]
    lib.kla_chunk_bwd.argtypes = [I, I, P, P, P, P, P, F, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, P]
    lib.kla_workspace_trim.argtypes = []
    for fn in ("kla_workspace_trim", "kla_chunk_fwd_noalloc", "kla_chunk_fwd", "kla_chunk_fwd_f32", "kla_chunk_fwd_ex", "kla_chunk_fwd_psd", "kla_plan", "kla_decode_step",
               "kla_decode_step_f32", "kla_decode_step_ex", "kla_loglinear_decode_step", "kla_loglinear_fwd",
               "kla_timing_enable",
               "kla_timing_select"):
        getattr(lib, fn).restype = I
    lib.kla_timing_enable.argtypes = [I]
    lib.kla_timing_select.argtypes = [ctypes.c_char_p]
    lib.kla_timing_collect.argtypes = [ctypes.POINTER(KernelTiming), I]
    lib.kla_timing_collect.restype = I
    lib.kla_last_error.restype = ctypes.c_char_p
    lib.kla_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def last_error() -> str:
    return load().kla_last_error().decode()


def version() -> str:
    return load().kla_version().decode()


def _check(status: int):
    if status != KLA_OK:
        raise KLAError(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, shape, dtypes, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.numel() and t.data_ptr() % 16:
        raise ValueError(f"{name} must start on a 16-byte boundary (a view with a storage offset is not)")


def chunk_fwd(q, k, v, log_alpha, eta, eps: float = 1e-6, init_state=None, chunk: int = 64,
              path: str = "auto", segments: int = 0, out=None, final_state=None,
              want_final: bool = True, stream=None, beta_mode: str = "kaczmarz") -> Tuple[object, Optional[object]]:
    """Chunkwise KLA prefill. q, k [B,T,H,dk] and v [B,T,H,dv] in bf16 (or all fp32);
    log_alpha, eta fp32 [B,T,H]; init_state fp32 [B,H,dk,dv] or None. beta_mode "kaczmarz"
    (KLA) or "direct" (beta = eta as given, the Gated DeltaNet rule).
    Returns (out fp32 [B,T,H,dv], final_state fp32 [B,H,dk,dv] or None)."""
    import torch
    lib = load()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype == torch.bfloat16:
        dtype = 0
    elif q.dtype == torch.float32:
        dtype = 1
    else:
        raise TypeError("q, k, v must be bfloat16 or float32")
    _need(q, "q", (B, T, H, dk), (q.dtype,), dev)
    _need(k, "k", (B, T, H, dk), (q.dtype,), dev)
    _need(v, "v", (B, T, H, dv), (q.dtype,), dev)
    _need(log_alpha, "log_alpha", (B, T, H), (torch.float32,), dev)
    _need(eta, "eta", (B, T, H), (torch.float32,), dev)
    if init_state is not None:
        _need(init_state, "init_state", (B, H, dk, dv), (torch.float32,), dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _need(out, "out", (B, T, H, dv), (torch.float32,), dev)
    if final_state is None and want_final:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", (B, H, dk, dv), (torch.float32,), dev)
    if path not in PATHS:
        raise ValueError(f"path must be one of {sorted(PATHS)}")
    if beta_mode not in BETA_MODES:
        raise ValueError(f"beta_mode must be one of {sorted(BETA_MODES)}")
    st = lib.kla_chunk_fwd_ex(dtype, BETA_MODES[beta_mode], _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(eta), float(eps),
                              _ptr(init_state), _ptr(out), _ptr(final_state), B, T, H, dk, dv, chunk,
                              PATHS[path], int(segments), _stream(stream))
    _check(st)
    return out, final_state


def chunk_fwd_noalloc(q, k, v, log_alpha, eta, eps: float = 1e-6, init_state=None, chunk: int = 64,
                      path: str = "auto", segments: int = 0, out=None, final_state=None, stream=None,
                      beta_mode: str = "kaczmarz"):
    """chunk_fwd through kla_chunk_fwd_noalloc: the workspace is the library's static device
    scratch buffer, so the call allocates no device memory (out and final_state must be given
    to avoid the binding's own allocations). Same results as chunk_fwd."""
    import torch
    lib = load()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    dtype = {torch.bfloat16: 0, torch.float32: 1}.get(q.dtype)
    if dtype is None:
        raise TypeError("q, k, v must be bfloat16 or float32")
    for t, n, shp in ((q, "q", (B, T, H, dk)), (k, "k", (B, T, H, dk)), (v, "v", (B, T, H, dv))):
        _need(t, n, shp, (q.dtype,), dev)
    _need(log_alpha, "log_alpha", (B, T, H), (torch.float32,), dev)
    _need(eta, "eta", (B, T, H), (torch.float32,), dev)
    if init_state is not None:
        _need(init_state, "init_state", (B, H, dk, dv), (torch.float32,), dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _need(out, "out", (B, T, H, dv), (torch.float32,), dev)
    if final_state is not None:
        _need(final_state, "final_state", (B, H, dk, dv), (torch.float32,), dev)
    if path not in PATHS or beta_mode not in BETA_MODES:
        raise ValueError("unknown path or beta_mode")
    _check(lib.kla_chunk_fwd_noalloc(dtype, BETA_MODES[beta_mode], _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                     _ptr(eta), float(eps), _ptr(init_state), _ptr(out), _ptr(final_state), B, T, H,
                                     dk, dv, chunk, PATHS[path], int(segments), _stream(stream)))
    return out, final_state


def chunk_fwd_psd(uq, uk, v, log_alpha, eta, eps: float = 1e-6, init_state=None, chunk: int = 64,
                  path: str = "auto", segments: int = 0, out=None, final_state=None,
                  want_final: bool = True, stream=None) -> Tuple[object, Optional[object]]:
    """Chunkwise KLA prefill with the rank-one PSD lift done in the kernels: uq, uk bf16
    [B,T,H,p] (p = 16), v bf16 [B,T,H,dv]; the kernels use q = psi(uq), k = psi(uk) with
    psi(u) = vec(u u^T) rounded to bf16 (dk = p*p). Other arguments as for chunk_fwd.
    Returns (out fp32 [B,T,H,dv], final_state fp32 [B,H,p*p,dv] or None)."""
    import torch
    lib = load()
    B, T, H, p = uq.shape
    dv = v.shape[-1]
    dk = p * p
    dev = uq.device
    _need(uq, "uq", (B, T, H, p), (torch.bfloat16,), dev)
    _need(uk, "uk", (B, T, H, p), (torch.bfloat16,), dev)
    _need(v, "v", (B, T, H, dv), (torch.bfloat16,), dev)
    _need(log_alpha, "log_alpha", (B, T, H), (torch.float32,), dev)
    _need(eta, "eta", (B, T, H), (torch.float32,), dev)
    if init_state is not None:
        _need(init_state, "init_state", (B, H, dk, dv), (torch.float32,), dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _need(out, "out", (B, T, H, dv), (torch.float32,), dev)
    if final_state is None and want_final:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if final_state is not None:
        _need(final_state, "final_state", (B, H, dk, dv), (torch.float32,), dev)
    if path not in PATHS:
        raise ValueError(f"path must be one of {sorted(PATHS)}")
    _check(lib.kla_chunk_fwd_psd(_ptr(uq), _ptr(uk), _ptr(v), _ptr(log_alpha), _ptr(eta), float(eps),
                                 _ptr(init_state), _ptr(out), _ptr(final_state), B, T, H, p, dv, chunk,
                                 PATHS[path], int(segments), _stream(stream)))
    return out, final_state


def decode_step(q, k, v, log_alpha, eta, state, eps: float = 1e-6, out=None, stream=None,
                beta_mode: str = "kaczmarz"):
    """One decode step for N x H states (updated in place). q, k [N,H,dk], v [N,H,dv] in bf16
    (or all fp32); log_alpha, eta fp32 [N,H]; state fp32 [N,H,dk,dv]; beta_mode as for
    chunk_fwd. Returns out fp32 [N,H,dv]."""
    import torch
    lib = load()
    N, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype == torch.bfloat16:
        dtype = 0
    elif q.dtype == torch.float32:
        dtype = 1
    else:
        raise TypeError("q, k, v must be bfloat16 or float32")
    if beta_mode not in BETA_MODES:
        raise ValueError(f"beta_mode must be one of {sorted(BETA_MODES)}")
    _need(k, "k", (N, H, dk), (q.dtype,), dev)
    _need(v, "v", (N, H, dv), (q.dtype,), dev)
    _need(q, "q", (N, H, dk), (q.dtype,), dev)
    _need(log_alpha, "log_alpha", (N, H), (torch.float32,), dev)
    _need(eta, "eta", (N, H), (torch.float32,), dev)
    _need(state, "state", (N, H, dk, dv), (torch.float32,), dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    _need(out, "out", (N, H, dv), (torch.float32,), dev)
    _check(lib.kla_decode_step_ex(dtype, BETA_MODES[beta_mode], _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                  _ptr(eta), float(eps), _ptr(state), _ptr(out), N, H, dk, dv, _stream(stream)))
    return out


def loglinear_decode_step(q, k, v, log_alpha, eta, lam, states, t: int, eps: float = 1e-6, out=None, stream=None,
                          beta_mode: str = "kaczmarz"):
    """Log-linear KLA decode of the token at position t for N x H heads. q, k [N,H,dk], v [N,H,dv]
    in bf16 (or all fp32); log_alpha, eta fp32 [N,H]; lam fp32 [N,H,L] (weight of each level in the
    output); states fp32 [N,H,L,dk,dv], the Fenwick buckets at position t-1, updated in place to
    position t. Returns out fp32 [N,H,dv]."""
    import torch
    lib = load()
    N, H, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    dev = q.device
    if q.dtype == torch.bfloat16:
        dtype = 0
    elif q.dtype == torch.float32:
        dtype = 1
    else:
        raise TypeError("q, k, v must be bfloat16 or float32")
    if beta_mode not in BETA_MODES:
        raise ValueError(f"beta_mode must be one of {sorted(BETA_MODES)}")
    _need(k, "k", (N, H, dk), (q.dtype,), dev)
    _need(v, "v", (N, H, dv), (q.dtype,), dev)
    _need(q, "q", (N, H, dk), (q.dtype,), dev)
    _need(log_alpha, "log_alpha", (N, H), (torch.float32,), dev)
    _need(eta, "eta", (N, H), (torch.float32,), dev)
    _need(lam, "lam", (N, H, L), (torch.float32,), dev)
    _need(states, "states", (N, H, L, dk, dv), (torch.float32,), dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=torch.float32, device=dev)
    _need(out, "out", (N, H, dv), (torch.float32,), dev)
    _check(lib.kla_loglinear_decode_step(dtype, BETA_MODES[beta_mode], _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                         _ptr(eta), _ptr(lam), float(eps), _ptr(states), _ptr(out), N, H, dk, dv,
                                         L, int(t), _stream(stream)))
    return out


def loglinear_fwd(q, k, v, log_alpha, eta, lam, eps: float = 1e-6, chunk: int = 64, out=None, stream=None,
                  beta_mode: str = "kaczmarz"):
    """Log-linear KLA prefill from empty buckets. q, k [B,T,H,dk], v [B,T,H,dv] in bf16 (or all
    fp32); log_alpha, eta fp32 [B,T,H]; lam fp32 [B,T,H,L] with T <= 2^(L-1).
    Returns out fp32 [B,T,H,dv]."""
    import torch
    lib = load()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    L = lam.shape[-1]
    dev = q.device
    if q.dtype == torch.bfloat16:
        dtype = 0
    elif q.dtype == torch.float32:
        dtype = 1
    else:
        raise TypeError("q, k, v must be bfloat16 or float32")
    if beta_mode not in BETA_MODES:
        raise ValueError(f"beta_mode must be one of {sorted(BETA_MODES)}")
    _need(q, "q", (B, T, H, dk), (q.dtype,), dev)
    _need(k, "k", (B, T, H, dk), (q.dtype,), dev)
    _need(v, "v", (B, T, H, dv), (q.dtype,), dev)
    _need(log_alpha, "log_alpha", (B, T, H), (torch.float32,), dev)
    _need(eta, "eta", (B, T, H), (torch.float32,), dev)
    _need(lam, "lam", (B, T, H, L), (torch.float32,), dev)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=torch.float32, device=dev)
    _need(out, "out", (B, T, H, dv), (torch.float32,), dev)
    _check(lib.kla_loglinear_fwd(dtype, BETA_MODES[beta_mode], _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha),
                                 _ptr(eta), _ptr(lam), float(eps), _ptr(out), B, T, H, dk, dv, L, chunk,
                                 _stream(stream)))
    return out


def chunk_bwd(q, k, v, log_alpha, eta, grad_out, eps: float = 1e-6, init_state=None, grad_final_state=None,
              chunk: int = 64, stream=None, beta_mode: str = "kaczmarz", want_grad_init: bool = True):
    """Gradients of the prefill for given d loss / d out (grad_out fp32 [B,T,H,dv]) and
    d loss / d final state (grad_final_state fp32 [B,H,dk,dv] or None: zero). Inputs as for
    chunk_fwd (dk in {64, 128}). Returns a dict of fp32 tensors: dq, dk [B,T,H,dk], dv [B,T,H,dv],
    dlog_alpha, deta [B,T,H] and dinit_state [B,H,dk,dv] (None unless want_grad_init)."""
    import torch
    lib = load()
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev = q.device
    if q.dtype == torch.bfloat16:
        dtype = 0
    elif q.dtype == torch.float32:
        dtype = 1
    else:
        raise TypeError("q, k, v must be bfloat16 or float32")
    if beta_mode not in BETA_MODES:
        raise ValueError(f"beta_mode must be one of {sorted(BETA_MODES)}")
    _need(q, "q", (B, T, H, dk), (q.dtype,), dev)
    _need(k, "k", (B, T, H, dk), (q.dtype,), dev)
    _need(v, "v", (B, T, H, dv), (q.dtype,), dev)
    _need(log_alpha, "log_alpha", (B, T, H), (torch.float32,), dev)
    _need(eta, "eta", (B, T, H), (torch.float32,), dev)
    _need(grad_out, "grad_out", (B, T, H, dv), (torch.float32,), dev)
    if init_state is not None:
        _need(init_state, "init_state", (B, H, dk, dv), (torch.float32,), dev)
    if grad_final_state is not None:
        _need(grad_final_state, "grad_final_state", (B, H, dk, dv), (torch.float32,), dev)
    f = dict(dtype=torch.float32, device=dev)
    g = dict(dq=torch.empty((B, T, H, dk), **f), dk=torch.empty((B, T, H, dk), **f),
             dv=torch.empty((B, T, H, dv), **f), dlog_alpha=torch.empty((B, T, H), **f),
             deta=torch.empty((B, T, H), **f),
             dinit_state=torch.empty((B, H, dk, dv), **f) if want_grad_init else None)
    _check(lib.kla_chunk_bwd(dtype, BETA_MODES[beta_mode], _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(eta),
                             float(eps), _ptr(init_state), _ptr(grad_out), _ptr(grad_final_state), _ptr(g["dq"]),
                             _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dlog_alpha"]), _ptr(g["deta"]),
                             _ptr(g["dinit_state"]), B, T, H, dk, dv, chunk, _stream(stream)))
    return g


def plan(B: int, T: int, H: int, dk: int, dv: int, chunk: int = 64, path: str = "auto",
         segments: int = 0, num_cus: int = 256, dtype: str = "bf16"):
    """Host-only: (path name, segments, workspace bytes) the library would use."""
    lib = load()
    p, s, w = ctypes.c_int(), ctypes.c_int(), ctypes.c_size_t()
    _check(lib.kla_plan(DTYPES[dtype], B, T, H, dk, dv, chunk, PATHS[path], segments, num_cus,
                        ctypes.byref(p), ctypes.byref(s), ctypes.byref(w)))
    return _PATH_NAMES[p.value], s.value, w.value


def workspace_trim():
    """Release the workspace the library's pool keeps reserved on the current device."""
    _check(load().kla_workspace_trim())


def timing_enable(enable: bool = True):
    _check(load().kla_timing_enable(1 if enable else 0))


def timing_select(kernel: Optional[str] = None):
    """Stamp only launches of `kernel` (None: every kernel) while the hook is on."""
    _check(load().kla_timing_select(kernel.encode() if kernel else None))


def timing_collect(max_kernels: int = 16):
    """{kernel name: (launches, total ms)} for launches timed since the last collect."""
    arr = (KernelTiming * max_kernels)()
    n = load().kla_timing_collect(arr, max_kernels)
    if n < 0:
        raise KLAError(KLA_ERR_HIP, last_error())
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(min(n, max_kernels))}
