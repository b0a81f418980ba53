"""kla_chunk_fwd_noalloc (static device scratch, no allocation) against kla_chunk_fwd_ex.

Both are called through the C ABI (ctypes) on the same seeded inputs, two calls in a
row with the second smaller, on both inter-chunk paths; the two entry points run the
same kernels with the same plan, so their outputs and end states must agree bit for bit.
A call whose workspace exceeds the scratch buffer is refused on the host.
"""
import ctypes
import sys

import numpy as np
import pytest

import workloads as W
from tests.gpu_common import upload_prefill

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import delta_rule_recurrence_kla_amd as kla  # noqa: E402


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _call(fn, wl, path, segments):
    q, k, v, la, eta, s0 = upload_prefill(wl)
    out = torch.full((wl.B, wl.T, wl.H, wl.dv), float("nan"), dtype=torch.float32, device="cuda:0")
    fin = torch.full((wl.B, wl.H, wl.dk, wl.dv), float("nan"), dtype=torch.float32, device="cuda:0")
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    dtype = 0 if wl.dtype == "bf16" else 1
    st = fn(dtype, 0, p(q), p(k), p(v), p(la), p(eta), float(wl.eps), p(s0), p(out), p(fin), wl.B, wl.T, wl.H, wl.dk,
            wl.dv, 64, kla.PATHS[path], segments, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0, kla.last_error()
    return out, fin


@pytest.mark.parametrize("path", ["sequential", "scan"])
@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("bf16", 256, 64), ("f32", 64, 128)])
def test_noalloc_matches_allocating_entry(path, dtype, dk, dv):
    lib = kla.load()
    name = "lm_layer_4k" if dtype == "bf16" else "tiny_f32"
    for i, (B, T, H) in enumerate([(3, 1000, 4), (2, 333, 3)]):  # the second call is smaller
        log(f"case: noalloc path={path} dtype={dtype} dk={dk} dv={dv} call {i} B={B} T={T} H={H}")
        wl = W.make_prefill(name, seed=17 + i, B=B, T=T, H=H, dk=dk, dv=dv, init_std=0.2)
        o_ref, f_ref = _call(lib.kla_chunk_fwd_ex, wl, path, 3)
        o, f = _call(lib.kla_chunk_fwd_noalloc, wl, path, 3)
        assert torch.equal(o, o_ref), f"call {i}: outputs differ"
        assert torch.equal(f, f_ref), f"call {i}: end states differ"
        assert torch.isfinite(o).all()


def test_noalloc_lm_layer_shape_fits():
    """The LM-layer prefill (B=8, T=4096, H=16, d=128) fits the scratch buffer; its outputs
    equal the allocating entry point's on every head."""
    lib = kla.load()
    wl = W.make_prefill("lm_layer_4k", seed=0)
    _, _, ws = kla.plan(wl.B, wl.T, wl.H, wl.dk, wl.dv)
    assert ws <= 128 << 20
    log("case: noalloc LM-layer shape")
    o_ref, f_ref = _call(lib.kla_chunk_fwd_ex, wl, "auto", 0)
    o, f = _call(lib.kla_chunk_fwd_noalloc, wl, "auto", 0)
    assert torch.equal(o, o_ref) and torch.equal(f, f_ref)


def test_noalloc_refuses_oversized_workspace():
    """A workspace beyond the scratch buffer is refused before anything is enqueued."""
    lib = kla.load()
    P = ctypes.c_void_p(0x1000)
    st = lib.kla_chunk_fwd_noalloc(0, 0, P, P, P, P, P, 1e-6, None, P, None, 64, 8192, 16, 128, 128, 64, 1, 0, None)
    assert st == 2 and "scratch" in kla.last_error()
