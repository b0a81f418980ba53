"""Checks of the seeded input generator (CPU)."""
import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10 ** rng.uniform(-30, 30, 100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, -3.0e38, 1e-40], np.float32)])
    ours = W.bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)
    np.testing.assert_array_equal(W.round_to_bf16(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_psd_lift_identity():
    """psi(u).psi(w) = (u.w)^2 and ||psi(u)|| = ||u||^2 (KATA page, section 2.2)."""
    rng = np.random.default_rng(1)
    u = rng.standard_normal((50, 16)).astype(np.float64)
    w = rng.standard_normal((50, 16)).astype(np.float64)
    pu, pw = W.psd_lift(u).astype(np.float64), W.psd_lift(w).astype(np.float64)
    np.testing.assert_allclose(np.sum(pu * pw, -1), np.sum(u * w, -1) ** 2, rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(np.linalg.norm(pu, axis=-1), np.sum(u * u, -1), rtol=1e-5)


def test_prefill_determinism_and_shapes():
    a = W.make_prefill("tiny_f32", seed=0)
    b = W.make_prefill("tiny_f32", seed=0)
    c = W.make_prefill("tiny_f32", seed=1)
    for f in ("q", "k", "v", "log_alpha", "eta"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
        assert not np.array_equal(getattr(a, f), getattr(c, f))
    assert a.q.shape == (1, 256, 2, 64) and a.v.shape == (1, 256, 2, 64)
    assert a.log_alpha.shape == (1, 256, 2) and a.init_state is None
    assert a.dtype == "f32" and a.eps == 1e-6


def test_tiny_moments():
    a = W.make_prefill("tiny_f32", seed=0, T=4096, H=4)
    assert abs(a.q.mean()) < 0.02 and abs(a.q.std() - 1) < 0.02
    assert abs(a.v.std() - 1) < 0.02
    lk = np.log(np.linalg.norm(a.k, axis=-1) / np.sqrt(64))  # ~ N(0, 0.5) plus chi noise
    assert abs(lk.std() - 0.5) < 0.06
    alpha = np.exp(a.log_alpha)
    assert 0.85 < alpha.mean() < 0.97 and alpha.max() < 1
    assert abs(a.eta.mean() - 0.5) < 0.02 and a.eta.min() > 0 and a.eta.max() < 1


def test_l2norm_recipe_bf16():
    a = W.make_prefill("lm_layer_4k", seed=0, B=1, T=256, H=4)
    assert a.dtype == "bf16"
    np.testing.assert_array_equal(W.round_to_bf16(a.q), a.q)
    ln = np.log(np.linalg.norm(a.k.astype(np.float64), axis=-1))
    assert abs(ln.mean()) < 0.05 and abs(ln.std() - 0.5) < 0.05


def test_psd_recipe():
    a = W.make_prefill("psd_lift_8k", seed=0, B=1, T=128, H=2)
    assert a.dk == 256 and a.q.shape[-1] == 256
    assert np.all(a.log_alpha == 0) and np.all(a.eta == 1)
    # unit u gives ||psi(u)|| = 1 up to bf16 rounding
    np.testing.assert_allclose(np.linalg.norm(a.k, axis=-1), 1.0, atol=1e-2)


def test_decode_inputs():
    s0 = W.make_decode_state(N=4, H=2, dk=16, dv=8)
    assert abs(s0.std() - 0.02) < 0.003
    st = W.make_decode_step(3, N=4, H=2, dk=16, dv=8)
    np.testing.assert_allclose(np.linalg.norm(st.k, axis=-1), 1.0, atol=1e-2)
    st2 = W.make_decode_step(3, N=4, H=2, dk=16, dv=8)
    np.testing.assert_array_equal(st.q, st2.q)
    many = W.make_decode_steps(4, N=4, H=2, dk=16, dv=8)
    np.testing.assert_array_equal(many.q[3], st.q)


def test_head_slice():
    a = W.make_prefill("tiny_f32", seed=0, H=3, B=2, T=64, init_std=0.1)
    s = a.head_slice([(1, 2), (0, 1)])
    np.testing.assert_array_equal(s.q[0, :, 0], a.q[1, :, 2])
    np.testing.assert_array_equal(s.init_state[1, 0], a.init_state[0, 1])


def test_psd_u_workload():
    """The PSD workload before the lift: the same unit vectors as the lifted recipe, in bf16."""
    a = W.make_psd_u(seed=0, B=2, T=50, H=3)
    b = W.make_psd_u(seed=0, B=2, T=50, H=3)
    np.testing.assert_array_equal(a.uq, b.uq)
    assert a.uq.shape == (2, 50, 3, 16) and a.v.shape == (2, 50, 3, 128)
    for x in (a.uq, a.uk, a.v):
        np.testing.assert_array_equal(x, W.round_to_bf16(x))          # bf16-exact values
    np.testing.assert_allclose(np.linalg.norm(a.uq, axis=-1), 1.0, atol=4e-3)
    assert np.all(a.log_alpha == 0) and np.all(a.eta == 1) and a.init_state is None
    lifted = W.make_prefill("psd_lift_8k", seed=0, B=2, T=50, H=3)
    # same draws in the same order: the lifted recipe's features are psi of the unrounded u
    np.testing.assert_allclose(W.psd_lift(a.uq), lifted.q, atol=2e-2)
    g = W.make_psd_u(seed=1, B=1, T=20, H=2, dv=64, gates="gaussian", init_std=0.5)
    assert np.all(g.log_alpha < 0) and np.all((g.eta > 0) & (g.eta < 1)) and g.init_state.shape == (1, 2, 256, 64)
    with pytest.raises(ValueError):
        W.make_psd_u(gates="other", B=1, T=1, H=1)


def test_loglinear_inputs():
    lam = W.make_loglinear_lambda(3, N=4, H=2, levels=5, seed=0)
    assert lam.shape == (4, 2, 5) and lam.dtype == np.float32 and np.all((lam > 0) & (lam < 1))
    np.testing.assert_array_equal(lam, W.make_loglinear_lambda(3, N=4, H=2, levels=5, seed=0))
    assert not np.array_equal(lam, W.make_loglinear_lambda(4, N=4, H=2, levels=5, seed=0))
    # the weights come from their own stream: the step's q, k, v are unchanged by drawing them
    st = W.make_decode_step(3, N=4, H=2, dk=8, dv=8, seed=0)
    np.testing.assert_array_equal(st.q, W.make_decode_step(3, N=4, H=2, dk=8, dv=8, seed=0).q)
    S = W.make_loglinear_states(N=2, H=2, levels=3, dk=4, dv=4, std=0.5, seed=1)
    assert S.shape == (2, 2, 3, 4, 4) and abs(float(S.std()) - 0.5) < 0.2
    cfg = W.LOGLINEAR_DECODE_CONFIG
    assert cfg["t0"] + cfg["steps"] <= 1 << (cfg["levels"] - 1)
