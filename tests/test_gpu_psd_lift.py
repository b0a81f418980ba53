"""GPU parity of the fused PSD lift (kla_chunk_fwd_psd) against the CPU oracle.

The kernels take the 16-wide u rows and form psi(u) = vec(u u^T) (KATA page, section
2.2), rounded to bf16, as they load each chunk. The oracle forms the same features in
float64 (oracle/psd_lift.py) and runs the token-by-token recurrence. Bar: the bf16 one,
max|err| <= 2e-2 * RMS(ref) on outputs and end state (the small cases use a tenth of it).
The fused path must also equal the unfused kernels on host-lifted features bit for bit:
both see the same bf16 features in the same order.
"""
import sys

import numpy as np
import pytest

import workloads as W
from oracle import cref, psd_lift
from tests.gpu_common import TOL, assert_close, err_over_rms, upload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import delta_rule_recurrence_kla_amd as kla  # noqa: E402


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _upload(wl):
    uq, uk, v = (upload(x, "bf16") for x in (wl.uq, wl.uk, wl.v))
    la, eta = upload(wl.log_alpha, "f32"), upload(wl.eta, "f32")
    s0 = None if wl.init_state is None else upload(wl.init_state, "f32")
    return uq, uk, v, la, eta, s0


def run_fused(wl, path="auto", segments=0, eps=None):
    uq, uk, v, la, eta, s0 = _upload(wl)
    out, fin = kla.chunk_fwd_psd(uq, uk, v, la, eta, wl.eps if eps is None else eps, init_state=s0, path=path,
                                 segments=segments)
    torch.cuda.synchronize()
    return out.cpu().numpy(), fin.cpu().numpy()


def oracle_heads(wl, heads):
    """Oracle outputs and end states of the listed (b, h) heads over the whole sequence."""
    pick = lambda a: np.stack([a[b, :, h] for b, h in heads])[:, :, None]
    q = psd_lift.psd_features(pick(wl.uq))
    k = psd_lift.psd_features(pick(wl.uk))
    s0 = None
    if wl.init_state is not None:
        s0 = np.stack([wl.init_state[b, h] for b, h in heads])[:, None]
    o, S = cref.forward(q, k, pick(wl.v), pick(wl.log_alpha[..., None])[..., 0],
                        pick(wl.eta[..., None])[..., 0], wl.eps, s0)
    return o, S


def all_heads(wl):
    return [(b, h) for b in range(wl.B) for h in range(wl.H)]


@pytest.mark.parametrize("T", [64, 200, 1000])
@pytest.mark.parametrize("dv", [64, 128])
@pytest.mark.parametrize("path", ["sequential", "scan"])
@pytest.mark.parametrize("gates", ["psd", "gaussian"])
def test_fused_small(T, dv, path, gates):
    log(f"psd fused T={T} dv={dv} path={path} gates={gates}")
    wl = W.make_psd_u(seed=T + dv, B=2, T=T, H=2, dv=dv, gates=gates, init_std=0.2)
    o, S = run_fused(wl, path=path, segments=3)
    heads = all_heads(wl)
    o_ref, S_ref = oracle_heads(wl, heads)
    got_o = np.stack([o[b, :, h] for b, h in heads])
    got_S = np.stack([S[b, h] for b, h in heads])
    assert_close(got_o, o_ref, TOL["bf16"] / 10, "out")
    assert_close(got_S, S_ref, TOL["bf16"] / 10, "final state")


@pytest.mark.parametrize("B,H,T", [(1, 1, 1), (1, 3, 65), (3, 5, 130)])
def test_fused_odd_grids(B, H, T):
    log(f"psd fused odd grid B={B} H={H} T={T}")
    wl = W.make_psd_u(seed=B * 100 + H * 10 + T, B=B, T=T, H=H, dv=128, gates="gaussian")
    o, S = run_fused(wl)
    heads = all_heads(wl)
    o_ref, S_ref = oracle_heads(wl, heads)
    assert_close(np.stack([o[b, :, h] for b, h in heads]), o_ref, TOL["bf16"] / 10, "out")
    assert_close(np.stack([S[b, h] for b, h in heads]), S_ref, TOL["bf16"] / 10, "final state")


@pytest.mark.parametrize("path", ["sequential", "scan"])
def test_fused_equals_unfused_on_lifted_features(path):
    """Same features, same kernels after the load: bit-identical outputs and end states."""
    log(f"psd fused == unfused path={path}")
    wl = W.make_psd_u(seed=11, B=2, T=64 * 9 + 17, H=3, dv=128, gates="gaussian", init_std=0.1)
    o_f, S_f = run_fused(wl, path=path, segments=4)
    uq, uk, v, la, eta, s0 = _upload(wl)
    q = upload(psd_lift.psd_features(wl.uq), "bf16")
    k = upload(psd_lift.psd_features(wl.uk), "bf16")
    o_u, S_u = kla.chunk_fwd(q, k, v, la, eta, wl.eps, init_state=s0, path=path, segments=4)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o_f, o_u.cpu().numpy())
    np.testing.assert_array_equal(S_f, S_u.cpu().numpy())


def test_fused_zero_length_copies_init():
    wl = W.make_psd_u(seed=2, B=2, T=0, H=2, dv=64, init_std=1.0)
    o, S = run_fused(wl)
    np.testing.assert_array_equal(S, wl.init_state)


def test_fused_exact_projection_self_check():
    """u_q = u_k with eta = 1, eps = 0: o_t = S_t^T k_t = v_t at every token (KLA page,
    "Theoretical derivation"), at the full PSD workload's length, without the oracle."""
    wl = W.make_psd_u(seed=9, B=1, T=8192, H=4, dv=128)
    wl.uq = wl.uk
    o, _ = run_fused(wl, eps=0.0)
    e = err_over_rms(o, wl.v)
    log(f"psd fused self-check max|o - v|/RMS(v) = {e:.2e}")
    assert e < 2e-2, e


def test_fused_full_size_sampled():
    """The full PSD workload (B=4, T=8192, H=8, p=16 -> 256 features, dv=128) in lifted form,
    sampled heads against the C oracle over all 8192 tokens, in the planner's path."""
    wl = W.make_psd_u(seed=0)
    log(f"psd fused full size B={wl.B} T={wl.T} H={wl.H} path={kla.plan(wl.B, wl.T, wl.H, 256, wl.dv)[:2]}")
    o, S = run_fused(wl)
    rng = np.random.default_rng(99)
    heads = sorted({(int(rng.integers(wl.B)), int(rng.integers(wl.H))) for _ in range(6)})
    o_ref, S_ref = oracle_heads(wl, heads)
    e1 = assert_close(np.stack([o[b, :, h] for b, h in heads]), o_ref, TOL["bf16"], "out")
    e2 = assert_close(np.stack([S[b, h] for b, h in heads]), S_ref, TOL["bf16"], "state")
    log(f"psd fused full size: out {e1:.2e} state {e2:.2e} on {len(heads)} heads")
