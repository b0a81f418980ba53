"""GPU parity of the log-linear KLA decode step (kla_loglinear_decode_step) against the
CPU oracle's recurrent form (oracle/loglinear.py).

Each case runs successive positions from a start position, comparing every step's output
and the occupied bucket states with the oracle. Bar: fp32 arithmetic on exact inputs, so
max|err| <= 1e-4 * RMS(ref) per step (the fp32 bar; the kernels' order of sums differs from
the oracle's); at full size, sampled heads at the bf16 bar.
"""
import sys

import numpy as np
import pytest

import workloads as W
from oracle import loglinear
from tests.gpu_common import TOL, assert_close, err_over_rms, upload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import delta_rule_recurrence_kla_amd as kla  # noqa: E402


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(N, H, dk, dv, L, t0, steps, dtype, beta_mode="kaczmarz", seed=0, std=0.3, heads=None, tol=1e-4,
         unit_weights=False):
    S0 = W.make_loglinear_states(N, H, L, dk, dv, std=std, seed=seed)
    S_dev = upload(S0, "f32")
    if heads is None:
        heads = [(n, h) for n in range(N) for h in range(H)]
    S_ref = np.stack([S0[n, h] for n, h in heads])[:, None].astype(np.float64)   # [n, 1, L, dk, dv]
    pick = lambda a: np.stack([a[n, h] for n, h in heads])[:, None]
    worst = 0.0
    for i in range(steps):
        t = t0 + i
        st = W.make_decode_step(i, N, H, dk, dv, dtype=dtype, seed=seed)
        lam = np.ones((N, H, L), np.float32) if unit_weights else W.make_loglinear_lambda(i, N, H, L, seed=seed)
        o = kla.loglinear_decode_step(upload(st.q, dtype), upload(st.k, dtype), upload(st.v, dtype),
                                      upload(st.log_alpha, "f32"), upload(st.eta, "f32"), upload(lam, "f32"),
                                      S_dev, t, st.eps, beta_mode=beta_mode)
        o_ref, S_ref = loglinear.decode_step_loglinear(S_ref, t, pick(st.q), pick(st.k), pick(st.v),
                                                       pick(st.log_alpha), pick(st.eta), pick(lam), st.eps,
                                                       beta_mode)
        og = o.cpu().numpy()
        got = np.stack([og[n, h] for n, h in heads])
        e = err_over_rms(got, o_ref[:, 0])
        worst = max(worst, e)
        assert np.all(np.isfinite(got)) and e <= tol, f"step t={t}: out max|err|/RMS = {e:.3e}"
    occ = loglinear.occupied_levels(t0 + steps - 1)
    Sg = S_dev.cpu().numpy()
    got_S = np.stack([Sg[n, h][occ] for n, h in heads])
    assert_close(got_S, S_ref[:, 0][:, occ], tol, "occupied bucket states")
    return worst


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (256, 128), (128, 64), (64, 128), (256, 64)])
def test_loglinear_from_empty(dtype, dk, dv):
    """Positions 0..69 from empty buckets (every merge pattern up to level 7)."""
    log(f"loglinear from empty dtype={dtype} dk={dk} dv={dv}")
    _run(N=2, H=3, dk=dk, dv=dv, L=8, t0=0, steps=70, dtype=dtype, std=0.0)


@pytest.mark.parametrize("t0", [1, 255, 1023, 32768 - 3])
def test_loglinear_from_positions(t0):
    """Start from filled buckets at positions whose next steps merge many levels at once
    (e.g. 1023 -> 1024 joins ten buckets), and at the top of a 16-level range."""
    log(f"loglinear from t0={t0}")
    _run(N=2, H=2, dk=128, dv=128, L=16, t0=t0, steps=3, dtype="bf16", seed=t0)


@pytest.mark.parametrize("beta_mode", ["kaczmarz", "direct"])
def test_loglinear_beta_modes(beta_mode):
    log(f"loglinear beta_mode={beta_mode}")
    _run(N=2, H=2, dk=64, dv=64, L=7, t0=5, steps=20, dtype="f32", beta_mode=beta_mode, std=0.1)


def test_unit_weights_match_kla_decode():
    """All-ones weights: the buckets sum to the KLA state, so outputs equal kla_decode_step's
    from the summed start state."""
    N, H, dk, dv, L, t0, steps = 3, 2, 128, 128, 10, 37, 12
    log("loglinear unit weights == KLA decode")
    S0 = W.make_loglinear_states(N, H, L, dk, dv, std=0.2, seed=4)
    occ = loglinear.occupied_levels(t0 - 1)
    S_dev = upload(S0, "f32")
    K_dev = upload(S0[:, :, occ].sum(axis=2), "f32")
    ones = upload(np.ones((N, H, L), np.float32), "f32")
    for i in range(steps):
        st = W.make_decode_step(i, N, H, dk, dv, dtype="bf16", seed=4)
        args = [upload(st.q, "bf16"), upload(st.k, "bf16"), upload(st.v, "bf16"), upload(st.log_alpha, "f32"),
                upload(st.eta, "f32")]
        o_ll = kla.loglinear_decode_step(*args, ones, S_dev, t0 + i, st.eps)
        o_k = kla.decode_step(*args, K_dev, st.eps)
        assert_close(o_ll.cpu().numpy(), o_k.cpu().numpy(), 1e-5, f"step {i}")
    occ = loglinear.occupied_levels(t0 + steps - 1)
    assert_close(S_dev.cpu().numpy()[:, :, occ].sum(axis=2), K_dev.cpu().numpy(), 1e-5, "summed buckets")


def test_loglinear_full_size_sampled():
    """256 sequences x 16 heads, dk=dv=128, 16 levels, 32 successive positions ending at
    32767 (up to 16 occupied buckets per head), sampled heads against the oracle."""
    cfg = W.LOGLINEAR_DECODE_CONFIG
    N, H, dk, dv, L = cfg["N"], cfg["H"], cfg["dk"], cfg["dv"], cfg["levels"]
    rng = np.random.default_rng(7)
    heads = sorted({(int(a), int(b)) for a, b in zip(rng.integers(0, N, 10), rng.integers(0, H, 10))})
    log(f"loglinear full size N={N} H={H} L={L} heads={len(heads)}")
    worst = _run(N=N, H=H, dk=dk, dv=dv, L=L, t0=32768 - 32, steps=32, dtype="bf16", std=cfg["state_std"],
                 heads=heads, tol=TOL["bf16"])
    log(f"loglinear full size worst max|err|/RMS = {worst:.2e}")


# ---------------------------------------------------------------------------
# prefill (kla_loglinear_fwd)
def _prefill_case(B, T, H, dk, dv, L, dtype, seed, beta_mode="kaczmarz"):
    recipe = "gaussian" if dtype == "f32" else "l2norm"
    wl = W.make_prefill("lm_layer_4k", seed=seed, recipe=recipe, B=B, T=T, H=H, dk=dk, dv=dv,
                        dtype=dtype)
    rng = np.random.default_rng(seed + 1)
    lam = rng.uniform(0.2, 1.5, (B, T, H, L)).astype(np.float32)
    return wl, lam


def _run_prefill(wl, lam, beta_mode="kaczmarz"):
    q, k, v = (upload(x, wl.dtype) for x in (wl.q, wl.k, wl.v))
    out = kla.loglinear_fwd(q, k, v, upload(wl.log_alpha, "f32"), upload(wl.eta, "f32"), upload(lam, "f32"), wl.eps,
                            beta_mode=beta_mode)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("bf16", 64, 64), ("bf16", 128, 64), ("bf16", 256, 64),
                                         ("f32", 64, 128), ("f32", 128, 128)])
@pytest.mark.parametrize("T", [1, 70, 300])
def test_loglinear_prefill_small(dtype, dk, dv, T):
    """Against the token-pair definition: T = 300 covers the intra-chunk levels and the scales
    of 1, 2 and 4 chunks, with a ragged last chunk."""
    log(f"loglinear prefill dtype={dtype} dk={dk} dv={dv} T={T}")
    wl, lam = _prefill_case(2, T, 2, dk, dv, 10, dtype, seed=T + dk + dv)
    o = _run_prefill(wl, lam)
    o_ref = loglinear.forward_loglinear(wl.q, wl.k, wl.v, wl.log_alpha, wl.eta, lam, wl.eps)
    assert_close(o, o_ref, 1e-4 if dtype == "f32" else TOL["bf16"] / 10, "out")


def test_loglinear_prefill_direct_mode():
    log("loglinear prefill direct mode")
    # keys of norm ~1 (the l2norm recipe) keep eta ||k||^2 below 2, so the direct writes stay bounded
    wl = W.make_prefill("lm_layer_4k", seed=3, recipe="l2norm", B=1, T=200, H=2, dk=64, dv=64, dtype="f32")
    lam = np.random.default_rng(4).uniform(0.2, 1.5, (1, 200, 2, 9)).astype(np.float32)
    wl.eta = (wl.eta * 0.3).astype(np.float32)
    o = _run_prefill(wl, lam, beta_mode="direct")
    o_ref = loglinear.forward_loglinear(wl.q, wl.k, wl.v, wl.log_alpha, wl.eta, lam, wl.eps, beta_mode="direct")
    assert_close(o, o_ref, 1e-4, "out")


def test_loglinear_prefill_unit_weights_equal_kla():
    """All-ones weights: the buckets sum to the KLA state, so the outputs are kla_chunk_fwd's."""
    log("loglinear prefill unit weights == KLA prefill")
    wl, _ = _prefill_case(2, 64 * 21 + 9, 3, 128, 128, 12, "bf16", seed=8)
    lam = np.ones((wl.B, wl.T, wl.H, 12), np.float32)
    o = _run_prefill(wl, lam)
    q, k, v = (upload(x, "bf16") for x in (wl.q, wl.k, wl.v))
    o_k, _ = kla.chunk_fwd(q, k, v, upload(wl.log_alpha, "f32"), upload(wl.eta, "f32"), wl.eps)
    torch.cuda.synchronize()
    # two GPU paths with their own split-bf16 rounding (each about 5e-4 of RMS from the oracle on
    # such inputs): the bf16 small-case bar
    assert_close(o, o_k.cpu().numpy(), TOL["bf16"] / 10, "out")


def _recurrent_reference(wl, lam, b, h, L):
    """One head by the oracle's recurrent form over every token."""
    dk, dv = wl.q.shape[-1], wl.v.shape[-1]
    S = np.zeros((1, 1, L, dk, dv))
    ref = np.zeros((wl.T, dv))
    for t in range(wl.T):
        pick = lambda a: a[b, t, h][None, None]
        o_t, S = loglinear.decode_step_loglinear(S, t, pick(wl.q), pick(wl.k), pick(wl.v),
                                                 wl.log_alpha[b, t, h][None, None], wl.eta[b, t, h][None, None],
                                                 lam[b, t, h][None, None], wl.eps)
        ref[t] = o_t[0, 0]
    return ref


def test_loglinear_prefill_uneven_work_per_workgroup():
    """24 heads over 52 chunks less a ragged 17 tokens: the intra-chunk kernel's workgroups take four or five chunks
    each, and the scale walks share a head's half-blocks out in runs of unequal length (five, then one, at the
    lowest scale). Two heads against the recurrent form over every token."""
    B, T, H, L = 1, 64 * 52 - 17, 24, 13
    log(f"loglinear prefill uneven work B={B} T={T} H={H} L={L}")
    wl = W.make_prefill("lm_layer_4k", seed=21, B=B, T=T, H=H)
    lam = np.random.default_rng(22).uniform(0.2, 1.5, (B, T, H, L)).astype(np.float32)
    o = _run_prefill(wl, lam)
    for b, h in [(0, 0), (0, 23)]:
        e = assert_close(o[b, :, h], _recurrent_reference(wl, lam, b, h, L), TOL["bf16"] / 10, f"head {(b, h)}")
        log(f"loglinear prefill uneven work head {(b, h)}: {e:.2e}")


def test_loglinear_prefill_full_size_sampled():
    """The LM-layer shape (B=8, T=4096, H=16, dk=dv=128) with 13 levels, sampled heads against
    the oracle's recurrent form over all 4096 tokens."""
    B, T, H, L = 8, 4096, 16, 13
    log(f"loglinear prefill full size B={B} T={T} H={H} L={L}")
    wl = W.make_prefill("lm_layer_4k", seed=0)
    rng = np.random.default_rng(11)
    lam = rng.uniform(0.2, 1.5, (B, T, H, L)).astype(np.float32)
    o = _run_prefill(wl, lam)
    heads = [(3, 5), (7, 14)]
    for b, h in heads:
        S = np.zeros((1, 1, L, 128, 128))
        ref = np.zeros((T, 128))
        for t in range(T):
            pick = lambda a: a[b, t, h][None, None]
            o_t, S = loglinear.decode_step_loglinear(S, t, pick(wl.q), pick(wl.k), pick(wl.v),
                                                     wl.log_alpha[b, t, h][None, None], wl.eta[b, t, h][None, None],
                                                     lam[b, t, h][None, None], wl.eps)
            ref[t] = o_t[0, 0]
        e = assert_close(o[b, :, h], ref, TOL["bf16"], f"head {(b, h)}")
        log(f"loglinear prefill full size head {(b, h)}: {e:.2e}")


@pytest.mark.parametrize("B,H,T,L", [(1, 1, 256, 9), (3, 5, 130, 9), (1, 2, 128, 8), (2, 1, 64 * 5, 10)])
def test_loglinear_prefill_edges(B, H, T, L):
    """T = 2^(L-1) exactly (the top level in use), a grid of 15 heads, one and two full scales, and a
    sequence of whole chunks with an odd number of half-blocks at the lowest scale."""
    log(f"loglinear prefill edges B={B} H={H} T={T} L={L}")
    wl, lam = _prefill_case(B, T, H, 64, 64, L, "bf16", seed=B * 1000 + H * 100 + T)
    o = _run_prefill(wl, lam)
    o_ref = loglinear.forward_loglinear(wl.q, wl.k, wl.v, wl.log_alpha, wl.eta, lam, wl.eps)
    assert_close(o, o_ref, TOL["bf16"] / 10, "out")
