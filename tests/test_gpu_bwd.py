"""GPU parity of the chunkwise backward (kla_chunk_bwd) against the gradient oracle
(oracle/kla_bwd.py: reverse mode through the token loop, pinned by finite differences).

Every gradient (dq, dk, dv, dlog_alpha, deta and the start state's) is compared element by
element with the oracle run in float64 on the same (bf16-exact or fp32) inputs. Bar: the
kernels compute in fp32 on exact inputs, so the forward's fp32 bar holds for every gradient:
max|err| <= 1e-4 * RMS(ref) per gradient and head.
"""
import sys

import numpy as np
import pytest

import workloads as W
from oracle import kla_bwd
from tests.gpu_common import err_over_rms, upload, upload_prefill

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import delta_rule_recurrence_kla_amd as kla  # noqa: E402

BAR = 1e-4
NAMES = ("dq", "dk", "dv", "dlog_alpha", "deta")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(wl, heads=None, beta_mode="kaczmarz", with_init=True, with_dfin=True, bar=BAR, seed=0):
    B, T, H = wl.q.shape[:3]
    dk, dv = wl.q.shape[-1], wl.v.shape[-1]
    d_out, d_fin = W.make_bwd_grads(B, T, H, dk, dv, seed=seed)
    q, k, v, la, eta, s0 = upload_prefill(wl)
    if not with_init:
        s0 = None
    g = kla.chunk_bwd(q, k, v, la, eta, upload(d_out, "f32"), eps=wl.eps, init_state=s0,
                      grad_final_state=upload(d_fin, "f32") if with_dfin else None, beta_mode=beta_mode)
    torch.cuda.synchronize()
    got = {n: t.cpu().numpy() for n, t in g.items() if t is not None}
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(H)]
    worst = {}
    for b, h in heads:
        f = lambda a: np.asarray(a[b, :, h], np.float64)
        S0 = None if (not with_init or wl.init_state is None) else wl.init_state[b, h]
        ref = kla_bwd.backward(f(wl.q), f(wl.k), f(wl.v), f(wl.log_alpha), f(wl.eta), wl.eps, f(d_out),
                               d_fin[b, h] if with_dfin else None, S0, beta_mode)
        for n in NAMES:
            e = err_over_rms(got[n][b, :, h], ref[n])
            worst[n] = max(worst.get(n, 0.0), e)
            assert np.all(np.isfinite(got[n][b, :, h])), f"{n} head {(b, h)}: non-finite"
            assert e <= bar, f"{n} head {(b, h)}: max|err|/RMS = {e:.3e} > {bar:.1e}"
        e = err_over_rms(got["dinit_state"][b, h], ref["dS0"])
        worst["dS0"] = max(worst.get("dS0", 0.0), e)
        assert e <= bar, f"dS0 head {(b, h)}: max|err|/RMS = {e:.3e} > {bar:.1e}"
    log("worst max|err|/RMS: " + ", ".join(f"{n} {e:.2e}" for n, e in worst.items()))
    return worst


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_bwd_several_chunks_ragged_tail(dtype, dk, dv):
    log(f"case: bwd dtype={dtype} dk={dk} dv={dv} T=200")
    wl = W.make_prefill("tiny_f32", seed=1, B=1, T=200, H=2, dk=dk, dv=dv, dtype=dtype, init_std=0.3)
    _run(wl)


def test_bwd_dk256_bf16():
    """dk = 256 (the PSD lift's feature width) in bf16, several chunks and a ragged tail."""
    log("case: bwd dtype=bf16 dk=256 dv=128 T=200")
    wl = W.make_prefill("tiny_f32", seed=9, B=1, T=200, H=2, dk=256, dv=128, dtype="bf16", init_std=0.3)
    _run(wl)


def test_bwd_psd_shape_full_size_prefix_gradient():
    """The PSD workload's shape (B=4, T=8192, H=8, dk=256 lifted features, dv=128, bf16), the
    whole call. The output gradient is zero past token 1024 and there is no end-state gradient,
    so every gradient past token 1024 is exactly zero and the first 1024 tokens' gradients (and
    the start state's) are those of the 1024-token prefix, which the oracle computes for one
    sampled head."""
    log("case: bwd psd_lift_8k full size, prefix 1024 of head (3,7)")
    wl = W.make_prefill("psd_lift_8k", seed=0, init_std=0.3)
    B, T, H, dk, dv, TP = wl.B, wl.T, wl.H, wl.dk, wl.dv, 1024
    d_out, _ = W.make_bwd_grads(B, T, H, dk, dv, seed=0)
    d_out[:, TP:] = 0.0
    q, k, v, la, eta, s0 = upload_prefill(wl)
    g = kla.chunk_bwd(q, k, v, la, eta, upload(d_out, "f32"), eps=wl.eps, init_state=s0)
    torch.cuda.synchronize()
    b, h = 3, 7
    f = lambda a: np.asarray(a[b, :TP, h], np.float64)
    ref = kla_bwd.backward(f(wl.q), f(wl.k), f(wl.v), f(wl.log_alpha), f(wl.eta), wl.eps, f(d_out), None,
                           wl.init_state[b, h], "kaczmarz")
    worst = {}
    for n in NAMES:
        got = g[n][b, :, h].cpu().numpy()
        assert not np.any(got[TP:]), f"{n}: nonzero past the gradient's support"
        e = err_over_rms(got[:TP], ref[n])
        worst[n] = e
        assert e <= BAR, f"{n}: max|err|/RMS = {e:.3e} > {BAR:.1e}"
    e = err_over_rms(g["dinit_state"][b, h].cpu().numpy(), ref["dS0"])
    worst["dS0"] = e
    assert e <= BAR, f"dS0: max|err|/RMS = {e:.3e} > {BAR:.1e}"
    log("worst max|err|/RMS: " + ", ".join(f"{n} {e:.2e}" for n, e in worst.items()))


@pytest.mark.parametrize("dk,dv,ends", [(128, 128, True), (64, 128, True), (128, 64, False)])
def test_bwd_segmented_walks(dk, dv, ends):
    """Two heads over 25 chunks (ragged tail): the planner segments this shape (few heads, long
    enough), so both walks run in segments from the forward scan's start states and the folded
    end gradients; every token and head against the oracle, with or without a start state and
    an end-state gradient."""
    log(f"case: bwd segmented walks dk={dk} dv={dv} B=1 H=2 T=1553 ends={ends}")
    wl = W.make_prefill("tiny_f32", seed=11, B=1, T=64 * 24 + 17, H=2, dk=dk, dv=dv, dtype="bf16", init_std=0.3)
    assert kla.plan(1, wl.T, 2, dk, dv)[0] == "scan"
    _run(wl, with_init=ends, with_dfin=ends)


def test_bwd_long_context_prefix_gradient():
    """The long-context shape (B=1, T=131072, H=16, dk=dv=128, bf16): 2048 chunks per walk on few
    heads. As in the PSD-shape test, the output gradient is zero past token 1024, so every later
    gradient must be exactly zero and the first 1024 tokens' gradients are those of the prefix."""
    log("case: bwd long_131k full size, prefix 1024 of head (0,9)")
    wl = W.make_prefill("long_131k", seed=0, init_std=0.3)
    B, T, H, dk, dv, TP = wl.B, wl.T, wl.H, wl.dk, wl.dv, 1024
    d_out = np.zeros((B, T, H, dv), np.float32)
    d_out[:, :TP] = W.make_bwd_grads(B, TP, H, dk, dv, seed=0)[0]
    q, k, v, la, eta, s0 = upload_prefill(wl)
    g = kla.chunk_bwd(q, k, v, la, eta, upload(d_out, "f32"), eps=wl.eps, init_state=s0)
    torch.cuda.synchronize()
    b, h = 0, 9
    f = lambda a: np.asarray(a[b, :TP, h], np.float64)
    ref = kla_bwd.backward(f(wl.q), f(wl.k), f(wl.v), f(wl.log_alpha), f(wl.eta), wl.eps, f(d_out), None,
                           wl.init_state[b, h], "kaczmarz")
    worst = {}
    for n in NAMES:
        got = g[n][b, :, h].cpu().numpy()
        assert not np.any(got[TP:]), f"{n}: nonzero past the gradient's support"
        e = err_over_rms(got[:TP], ref[n])
        worst[n] = e
        assert e <= BAR, f"{n}: max|err|/RMS = {e:.3e} > {BAR:.1e}"
    e = err_over_rms(g["dinit_state"][b, h].cpu().numpy(), ref["dS0"])
    worst["dS0"] = e
    assert e <= BAR, f"dS0: max|err|/RMS = {e:.3e} > {BAR:.1e}"
    log("worst max|err|/RMS: " + ", ".join(f"{n} {e:.2e}" for n, e in worst.items()))


@pytest.mark.parametrize("T", [1, 63, 64, 65, 128])
def test_bwd_chunk_edges(T):
    log(f"case: bwd edges T={T}")
    wl = W.make_prefill("tiny_f32", seed=2, B=2, T=T, H=1, init_std=0.3)
    _run(wl)


def test_bwd_without_start_state_or_end_gradient():
    log("case: bwd no init, no dS_T")
    wl = W.make_prefill("tiny_f32", seed=3, T=150)
    _run(wl, with_init=False, with_dfin=False)


def test_bwd_direct_write_strength():
    log("case: bwd direct mode")
    wl = W.make_prefill("tiny_f32", seed=4, T=190, recipe="l2norm", init_std=0.3)
    _run(wl, beta_mode="direct")


def test_bwd_growth_gates():
    """log_alpha > 0 in places (e^{g_r - g_i} > 1 inside a chunk)."""
    log("case: bwd growth gates")
    wl = W.make_prefill("tiny_f32", seed=5, T=160, init_std=0.3)
    wl.log_alpha[:] = np.random.default_rng(5).uniform(-0.05, 0.04, wl.log_alpha.shape).astype(np.float32)
    _run(wl)


def test_bwd_zero_tokens_passes_the_end_gradient_through():
    log("case: bwd T=0")
    B, H, dk, dv = 2, 3, 64, 64
    _, d_fin = W.make_bwd_grads(B, 0, H, dk, dv, seed=6)
    e = lambda *s: torch.empty(s, dtype=torch.float32, device="cuda")
    q = torch.empty((B, 0, H, dk), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((B, 0, H, dv), dtype=torch.bfloat16, device="cuda")
    g = kla.chunk_bwd(q, q, v, e(B, 0, H), e(B, 0, H), e(B, 0, H, dv), grad_final_state=upload(d_fin, "f32"))
    np.testing.assert_array_equal(g["dinit_state"].cpu().numpy(), d_fin)


def test_bwd_lm_layer_full_size_sampled_heads():
    """B=8, T=4096, H=16, dk=dv=128 in bf16: the whole call, two heads checked in full."""
    log("case: bwd lm_layer_4k full size, heads (0,0) and (7,15)")
    wl = W.make_prefill("lm_layer_4k", seed=0, init_std=0.3)
    _run(wl, heads=[(0, 0), (7, 15)])


def test_bwd_odd_batch_and_heads():
    """B=3, H=5 (B*H not a multiple of the XCD count or of the column groups), bf16, dk=64, dv=128."""
    log("case: bwd B=3 H=5 T=130 dk=64 dv=128 bf16")
    wl = W.make_prefill("tiny_f32", seed=7, B=3, T=130, H=5, dk=64, dv=128, dtype="bf16", init_std=0.3)
    _run(wl, heads=[(0, 0), (1, 3), (2, 4)])


@pytest.mark.parametrize("B", [2, 4])
def test_bwd_walk_workgroup_sizes(B):
    """The walks take one-wave (B=2: 32 heads) or two-wave (B=4: 64 heads) workgroups when
    four-wave ones would not give every CU one; the LM-layer test covers four waves."""
    log(f"case: bwd lm_layer heads, B={B} T=300")
    wl = W.make_prefill("lm_layer_4k", seed=10, B=B, T=300, init_std=0.3)
    _run(wl, heads=[(0, 0), (B - 1, 15)])


def test_bwd_repeat_calls_are_bit_identical():
    """No atomics or order-dependent reductions: two calls on the same inputs agree bit for bit."""
    log("case: bwd determinism, lm_layer shape with B=2")
    wl = W.make_prefill("lm_layer_4k", seed=8, B=2, T=1000, init_std=0.3)
    d_out, d_fin = W.make_bwd_grads(2, 1000, wl.H, wl.dk, wl.dv, seed=8)
    q, k, v, la, eta, s0 = upload_prefill(wl)
    args = (q, k, v, la, eta, upload(d_out, "f32"))
    g1 = kla.chunk_bwd(*args, eps=wl.eps, init_state=s0, grad_final_state=upload(d_fin, "f32"))
    g2 = kla.chunk_bwd(*args, eps=wl.eps, init_state=s0, grad_final_state=upload(d_fin, "f32"))
    torch.cuda.synchronize()
    for n in g1:
        assert torch.equal(g1[n], g2[n]), n
