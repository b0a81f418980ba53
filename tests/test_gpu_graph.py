"""Decode steps, and the allocation-free prefill, captured in a HIP graph (through
torch.cuda.graph) replay exactly what the eager calls compute. Decode and
kla_chunk_fwd_noalloc allocate nothing, so a serving loop can capture a run of calls and
replay it without per-launch host overhead. Each replay starts from a state reset by an
eager copy (or outputs overwritten eagerly), and every replay is checked against the eager
results, bit for bit (same kernels, same inputs)."""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import delta_rule_recurrence_kla_amd as kla  # noqa: E402
from tests.gpu_common import upload  # noqa: E402


def _steps(n, N, H, dk, dv, seed):
    out = []
    for s in range(n):
        st = W.make_decode_step(s, N, H, dk, dv, dtype="bf16", seed=seed)
        out.append((upload(st.q, "bf16"), upload(st.k, "bf16"), upload(st.v, "bf16"), upload(st.log_alpha, "f32"),
                    upload(st.eta, "f32")))
    return out


def test_decode_graph_replays_match_eager():
    N, H, dk, dv, n = 8, 4, 128, 128, 12
    S0 = upload(W.make_decode_state(N, H, dk, dv, std=0.1, seed=5), "f32")
    ins = _steps(n, N, H, dk, dv, seed=5)
    S_e = S0.clone()
    eager = [kla.decode_step(*ins[s], S_e, 1e-6).clone() for s in range(n)]
    torch.cuda.synchronize()

    S_g = S0.clone()
    outs = [torch.empty((N, H, dv), dtype=torch.float32, device=S0.device) for _ in range(n)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture, on a scratch state
        kla.decode_step(*ins[0], S0.clone(), 1e-6)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(n):
            kla.decode_step(*ins[s], S_g, 1e-6, out=outs[s])
    for rep in range(3):
        S_g.copy_(S0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(n):
            assert torch.equal(outs[s], eager[s]), f"replay {rep}, step {s}"
        assert torch.equal(S_g, S_e), f"replay {rep}: state"


def test_loglinear_decode_graph_replays_match_eager():
    N, H, dk, dv, L, t0, n = 4, 2, 128, 128, 8, 60, 10
    S0 = upload(W.make_loglinear_states(N, H, L, dk, dv, std=0.1, seed=6), "f32")
    ins = _steps(n, N, H, dk, dv, seed=6)
    lam = [upload(W.make_loglinear_lambda(s, N, H, L, seed=6), "f32") for s in range(n)]
    S_e = S0.clone()
    eager = [kla.loglinear_decode_step(*ins[s], lam[s], S_e, t0 + s, 1e-6).clone() for s in range(n)]
    torch.cuda.synchronize()

    S_g = S0.clone()
    outs = [torch.empty((N, H, dv), dtype=torch.float32, device=S0.device) for _ in range(n)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        kla.loglinear_decode_step(*ins[0], lam[0], S0.clone(), t0, 1e-6)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for s in range(n):
            kla.loglinear_decode_step(*ins[s], lam[s], S_g, t0 + s, 1e-6, out=outs[s])
    for rep in range(3):
        S_g.copy_(S0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s in range(n):
            assert torch.equal(outs[s], eager[s]), f"replay {rep}, step {s}"
        assert torch.equal(S_g, S_e), f"replay {rep}: buckets"


@pytest.mark.parametrize("path,segments", [("sequential", 0), ("scan", 3)])
def test_noalloc_prefill_graph_replays_match_eager(path, segments):
    """The allocation-free prefill (kla_chunk_fwd_noalloc: its workspace is the library's static
    device scratch) captured in a HIP graph on both inter-chunk paths: every replay, with eager
    work on the outputs between replays, matches the eager call bit for bit."""
    from tests.gpu_common import upload_prefill
    wl = W.make_prefill("tiny_f32", seed=12, B=2, T=64 * 6 + 9, H=3, dk=128, dv=128, dtype="bf16", init_std=0.2)
    q, k, v, la, eta, s0 = upload_prefill(wl)
    shp_o, shp_s = (wl.B, wl.T, wl.H, wl.dv), (wl.B, wl.H, wl.dk, wl.dv)
    f32 = dict(dtype=torch.float32, device=q.device)
    out_e, fin_e = torch.empty(shp_o, **f32), torch.empty(shp_s, **f32)
    kla.chunk_fwd_noalloc(q, k, v, la, eta, wl.eps, init_state=s0, path=path, segments=segments, out=out_e,
                          final_state=fin_e)
    torch.cuda.synchronize()

    out_g, fin_g = torch.empty(shp_o, **f32), torch.empty(shp_s, **f32)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture
        kla.chunk_fwd_noalloc(q, k, v, la, eta, wl.eps, init_state=s0, path=path, segments=segments, out=out_g,
                              final_state=fin_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kla.chunk_fwd_noalloc(q, k, v, la, eta, wl.eps, init_state=s0, path=path, segments=segments, out=out_g,
                              final_state=fin_g)
    for rep in range(3):
        out_g.fill_(float("nan"))
        fin_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {rep}: outputs"
        assert torch.equal(fin_g, fin_e), f"replay {rep}: end state"
