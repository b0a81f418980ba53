"""Helpers for the GPU parity tests: upload seeded workloads, compare with the oracle."""
import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def torch_dev():
    import torch
    return torch.device("cuda:0")


def upload(a, dtype):
    """float32 numpy array -> cuda tensor of `dtype` ('bf16' values are already bf16-exact)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch_dev())
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def upload_prefill(wl):
    import torch
    q, k, v = (upload(x, wl.dtype) for x in (wl.q, wl.k, wl.v))
    la = upload(wl.log_alpha, "f32")
    eta = upload(wl.eta, "f32")
    s0 = None if wl.init_state is None else upload(wl.init_state, "f32")
    return q, k, v, la, eta, s0


def err_over_rms(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2))
    return float(np.max(np.abs(got - ref)) / max(rms, 1e-300))


def assert_close(got, ref, tol, what):
    e = err_over_rms(got, ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert e <= tol, f"{what}: max|err|/RMS = {e:.3e} > {tol:.1e}"
    return e


def hip_runtime():
    """ctypes handle of the HIP runtime loaded in this process (the one torch and libkla use).
    A plain CDLL("libamdhip64.so") may load a second, separate copy of the runtime."""
    import ctypes
    import torch
    torch.cuda.init()
    for line in open("/proc/self/maps"):
        path = line.split()[-1] if len(line.split()) >= 6 else ""
        if "libamdhip64.so" in path:
            return ctypes.CDLL(path)
    raise RuntimeError("no HIP runtime loaded")
