"""C-ABI boundary checks that need no GPU: the library loads, exports every
function include/kla.h declares, rejects bad arguments before touching HIP, and
plans paths and workspaces as documented. No call here reaches a kernel."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kla.h")

kla = pytest.importorskip("delta_rule_recurrence_kla_amd")
if not os.path.exists(kla.lib_path()):
    pytest.skip("libkla.so not built", allow_module_level=True)

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kla_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("kla_chunk_fwd", "kla_chunk_fwd_f32", "kla_chunk_fwd_ex", "kla_chunk_fwd_psd", "kla_loglinear_decode_step",
              "kla_loglinear_fwd", "kla_chunk_bwd",
              "kla_decode_step", "kla_decode_step_ex",
              "kla_decode_step_f32", "kla_plan", "kla_last_error", "kla_version",
              "kla_timing_enable", "kla_timing_collect", "kla_timing_select", "kla_workspace_trim"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = kla.load()
    for n in _declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", kla.lib_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (kla_\w+)$", out, flags=re.M))
    assert set(_declared_functions()) <= exported


def test_timing_select_rejects_long_names():
    with pytest.raises(kla.KLAError):
        kla.timing_select("k" * 32)
    kla.timing_select("kla_state_seq")
    kla.timing_select(None)


def test_version_and_empty_error():
    assert "gfx950" in kla.version()
    assert isinstance(kla.last_error(), str)


def _chunk(lib, dtype=0, beta=0, q=FAKE, out=FAKE, B=1, T=64, H=1, dk=64, dv=64, chunk=64, path=0, segs=0):
    return lib.kla_chunk_fwd_ex(dtype, beta, q, FAKE, FAKE, FAKE, FAKE, 1e-6, None, out, None,
                                B, T, H, dk, dv, chunk, path, segs, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 1), (dict(H=0), 1), (dict(T=-1), 1), (dict(q=None), 1), (dict(out=None), 1),
    (dict(dk=96), 2), (dict(dv=256), 2), (dict(chunk=32), 2), (dict(dtype=7), 1),
    (dict(dtype=1, dk=256), 2), (dict(path=5), 1), (dict(segs=-1), 1), (dict(B=70000, H=1), 2),
    (dict(beta=2), 1), (dict(beta=-1), 1),
])
def test_prefill_validation(kw, status):
    lib = kla.load()
    assert _chunk(lib, **kw) == status
    assert kla.last_error() != ""


def _psd(lib, uq=FAKE, out=FAKE, B=1, T=64, H=1, p=16, dv=64, chunk=64, path=0, segs=0):
    return lib.kla_chunk_fwd_psd(uq, FAKE, FAKE, FAKE, FAKE, 1e-6, None, out, None, B, T, H, p, dv, chunk, path,
                                 segs, None)


@pytest.mark.parametrize("kw,status", [
    (dict(p=0), 1), (dict(p=8), 2), (dict(p=12), 2), (dict(p=32), 2), (dict(B=0), 1), (dict(T=-1), 1),
    (dict(uq=None), 1), (dict(out=None), 1), (dict(dv=96), 2), (dict(chunk=16), 2), (dict(path=3), 1),
    (dict(segs=-2), 1),
])
def test_psd_validation(kw, status):
    lib = kla.load()
    assert _psd(lib, **kw) == status
    assert kla.last_error() != ""


def test_psd_zero_tokens_without_final_state_is_a_no_op():
    lib = kla.load()
    assert _psd(lib, uq=None, out=None, T=0) == 0


def _ll(lib, dtype=0, beta=0, q=FAKE, lam=FAKE, N=2, H=2, dk=128, dv=128, L=16, t=5):
    return lib.kla_loglinear_decode_step(dtype, beta, q, FAKE, FAKE, FAKE, FAKE, lam, 1e-6, FAKE, FAKE, N, H, dk, dv,
                                         L, t, None)


@pytest.mark.parametrize("kw,status", [
    (dict(L=0), 1), (dict(L=32), 1), (dict(t=-1), 1), (dict(L=4, t=8), 1), (dict(L=1, t=1), 1),
    (dict(dk=100), 2), (dict(dv=32), 2), (dict(q=None), 1), (dict(lam=None), 1), (dict(dtype=5), 1),
    (dict(beta=3), 1), (dict(N=-1), 1), (dict(H=0), 1),
])
def test_loglinear_validation(kw, status):
    lib = kla.load()
    assert _ll(lib, **kw) == status
    assert kla.last_error() != ""


def _llf(lib, dtype=0, q=FAKE, lam=FAKE, B=1, T=64, H=1, dk=64, dv=64, L=8, chunk=64):
    return lib.kla_loglinear_fwd(dtype, 0, q, FAKE, FAKE, FAKE, FAKE, lam, 1e-6, FAKE, B, T, H, dk, dv, L, chunk, None)


@pytest.mark.parametrize("kw,status", [
    (dict(L=0), 1), (dict(L=32), 1), (dict(T=65, L=7), 1), (dict(T=129, L=8), 1), (dict(q=None), 1),
    (dict(lam=None), 1), (dict(dk=96), 2), (dict(dv=256), 2), (dict(chunk=32), 2), (dict(dtype=1, dk=256), 2),
    (dict(B=0), 1), (dict(T=-1), 1),
])
def test_loglinear_prefill_validation(kw, status):
    lib = kla.load()
    assert _llf(lib, **kw) == status
    assert kla.last_error() != ""


def test_loglinear_prefill_zero_tokens_is_a_no_op():
    lib = kla.load()
    assert _llf(lib, q=None, lam=None, T=0, L=1) == 0


def test_loglinear_zero_sequences_is_a_no_op():
    lib = kla.load()
    assert _ll(lib, q=None, lam=None, N=0, L=31, t=(1 << 30) - 1) == 0
    assert _ll(lib, q=None, lam=None, N=0, L=1, t=0) == 0


@pytest.mark.parametrize("args,status", [
    (dict(N=-1), 1), (dict(H=0), 1), (dict(dk=100), 2), (dict(dv=32), 2), (dict(q=None), 1),
    (dict(state=None), 1),
])
def test_decode_validation(args, status):
    lib = kla.load()
    a = dict(q=FAKE, state=FAKE, N=4, H=2, dk=128, dv=128)
    a.update(args)
    st = lib.kla_decode_step(a["q"], FAKE, FAKE, FAKE, FAKE, 1e-6, a["state"], FAKE,
                             a["N"], a["H"], a["dk"], a["dv"], None)
    assert st == status


@pytest.mark.parametrize("dtype,beta,status", [(0, 2, 1), (7, 0, 1), (1, 1, 0), (0, 1, 0)])
def test_decode_ex_validation(dtype, beta, status):
    lib = kla.load()
    # N = 0: validated, then nothing to do (no device access)
    assert lib.kla_decode_step_ex(dtype, beta, None, None, None, None, None, 1e-6, None, None, 0, 4, 128, 128,
                                  None) == status


def test_decode_zero_sequences_is_a_no_op():
    lib = kla.load()
    assert lib.kla_decode_step(None, None, None, None, None, 1e-6, None, None, 0, 4, 128, 128, None) == 0


def test_forced_workspace_failure(monkeypatch):
    """The OOM path returns KLA_ERR_OOM before any HIP call (forced from the host)."""
    monkeypatch.setenv("KLA_TEST_FAIL_ALLOC", "1")
    lib = kla.load()
    assert _chunk(lib) == 4
    assert "KLA_TEST_FAIL_ALLOC" in kla.last_error()


def test_plan_paths():
    # 0.4B-LM-shaped layer: B*H = 128 heads x 2 column groups fill 256 CUs -> sequential
    p, s, w = kla.plan(8, 4096, 16, 128, 128, num_cus=256)
    assert p == "sequential" and s == 1
    assert w >= 8 * 16 * 64 * 13056                      # compact bf16 record
    assert kla.plan(8, 4096, 16, 128, 128, num_cus=256, dtype="f32")[2] >= 8 * 16 * 64 * 33536
    # long context with 16 heads under-fills the chip -> scan with several segments
    p, s, w = kla.plan(1, 131072, 16, 128, 128, num_cus=256)
    assert p == "scan" and 4 <= s <= 64
    # the segment counts that measured fastest on 256 CUs (sweeps over 2..32 segments): 8 for the
    # 131K-token shape; 4 for the PSD shape, whose map walk then fits one round at two
    # workgroups per CU once segment 0's identity columns are skipped
    assert kla.plan(1, 131072, 16, 128, 128, num_cus=256)[:2] == ("scan", 8)
    assert kla.plan(4, 8192, 8, 256, 128, num_cus=256)[:2] == ("scan", 4)
    # explicit choices are honoured; segments are clamped so that none is empty
    assert kla.plan(1, 131072, 16, 128, 128, path="sequential", num_cus=256)[:2] == ("sequential", 1)
    p, s, _ = kla.plan(1, 64 * 10, 1, 64, 64, path="scan", segments=4, num_cus=256)
    assert p == "scan" and s == 4
    p, s, _ = kla.plan(1, 64 * 10, 1, 64, 64, path="scan", segments=100, num_cus=256)
    assert p == "scan" and s == 10
    # a single chunk cannot be split
    assert kla.plan(1, 64, 1, 64, 64, path="scan", num_cus=256)[:2] == ("sequential", 1)
    assert kla.plan(2, 0, 2, 64, 64, num_cus=256)[1:] == (1, 0)


@pytest.mark.parametrize("dtype,dk,rec_bytes", [("bf16", 128, 13056), ("bf16", 256, 33536), ("f32", 128, 33536)])
def test_plan_workspace_bytes(dtype, dk, rec_bytes):
    """Workspace = chunk records + segment maps + segment start states, each 256-byte aligned.
    bf16 with dk <= 128 uses the compact record (no P, T' without its zero quadrant)."""
    _, s, w = kla.plan(1, 64 * 10, 2, dk, 64, path="scan", segments=5, num_cus=256, dtype=dtype)
    rec = 2 * 10 * rec_bytes
    maps = 2 * 4 * dk * (dk + 64) * 4
    starts = 2 * 5 * dk * 64 * 4
    up = lambda x: (x + 255) // 256 * 256
    assert w == up(rec) + up(maps) + up(starts)


def _bwd(lib, dtype=0, beta=0, q=FAKE, dout=FAKE, gq=FAKE, ginit=None, B=1, T=64, H=1, dk=64, dv=64, chunk=64):
    return lib.kla_chunk_bwd(dtype, beta, q, FAKE, FAKE, FAKE, FAKE, 1e-6, None, dout, None, gq, FAKE, FAKE, FAKE,
                             FAKE, ginit, B, T, H, dk, dv, chunk, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(dout=None), 1), (dict(gq=None), 1), (dict(dtype=7), 1), (dict(beta=4), 1),
    (dict(B=0), 1), (dict(T=-1), 1), (dict(dk=256, dtype=1), 2), (dict(dk=96), 2), (dict(dv=32), 2), (dict(chunk=128), 2),
])
def test_bwd_validation(kw, status):
    lib = kla.load()
    assert _bwd(lib, **kw) == status
    assert kla.last_error() != ""


def test_bwd_zero_tokens_without_start_gradient_is_a_no_op():
    lib = kla.load()
    assert _bwd(lib, q=None, dout=None, gq=None, T=0) == 0


MIS = ctypes.c_void_p(0x1008)  # 8-byte aligned only: rejected before any HIP call


@pytest.mark.parametrize("call", [
    lambda lib: lib.kla_chunk_fwd_ex(0, 0, MIS, FAKE, FAKE, FAKE, FAKE, 1e-6, None, FAKE, None, 1, 64, 1, 64, 64, 64,
                                     0, 0, None),
    lambda lib: lib.kla_chunk_fwd_ex(0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, MIS, FAKE, None, 1, 64, 1, 64, 64, 64,
                                     0, 0, None),
    lambda lib: lib.kla_chunk_fwd_ex(1, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, None, FAKE, MIS, 1, 64, 1, 64, 64, 64,
                                     0, 0, None),
    lambda lib: lib.kla_chunk_fwd_psd(FAKE, MIS, FAKE, FAKE, FAKE, 1e-6, None, FAKE, None, 1, 64, 1, 16, 64, 64, 0, 0,
                                      None),
    lambda lib: lib.kla_decode_step(FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, MIS, FAKE, 4, 2, 128, 128, None),
    lambda lib: lib.kla_decode_step_f32(FAKE, FAKE, FAKE, MIS, FAKE, 1e-6, FAKE, FAKE, 4, 2, 128, 128, None),
    lambda lib: lib.kla_loglinear_decode_step(0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, MIS, 1e-6, FAKE, FAKE, 2, 2, 128,
                                              128, 16, 5, None),
    lambda lib: lib.kla_loglinear_fwd(0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, MIS, 1, 64, 1, 64, 64, 8, 64,
                                      None),
    lambda lib: lib.kla_chunk_bwd(0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, None, FAKE, None, FAKE, FAKE, FAKE, MIS,
                                  FAKE, None, 1, 64, 1, 64, 64, 64, None),
])
def test_misaligned_arrays_are_rejected(call):
    """kla.h: every array pointer is 16-byte aligned; a view with a storage offset is refused
    on the host with KLA_ERR_INVALID_ARG, before anything is enqueued."""
    lib = kla.load()
    assert call(lib) == 1
    assert "16-byte" in kla.last_error()


def test_binding_refuses_offset_views():
    torch = pytest.importorskip("torch")
    base = torch.zeros(16, dtype=torch.float32)
    with pytest.raises(ValueError, match="16-byte"):
        kla._need(base[1:9], "x", (8,), (torch.float32,), base.device)
    kla._need(base[4:12], "x", (8,), (torch.float32,), base.device)  # 16 bytes in: accepted
