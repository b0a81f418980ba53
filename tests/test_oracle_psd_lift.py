"""Pins of the PSD-lift oracle (oracle/psd_lift.py) against what the pages and the
mathematics fix, and planted mistakes that the pins must catch (CPU only).

  rounding         hand-derived bf16 values: below half an ulp, and the two kinds of
                   exact tie (one rounds up to the even neighbour, one down)
  lift identities  psi(u).psi(w) = (u.w)^2 and ||psi(u)|| = ||u||^2 (KATA page, 2.2) on
                   inputs whose features are exact in bf16; psi(e_a + e_b) in closed form
  orthonormal      one-hot u_k give orthonormal lifted keys, where the delta rule reduces
                   to the masked parallel form (Log-Linear page, "Mathematical
                   formalization") with (u_q . e_a)^2 as the query-key product
  constraint       u_q = u_k, eta = 1, eps = 0: o_t = S_t^T k_t = v_t (KLA page, "KLA
                   update rule" at full step)
"""
import numpy as np
import pytest

from oracle import kla_ref, psd_lift

P = 16


def _dyadic(rng, shape, bits=3):
    """Values m / 2^bits with |m| <= 7: every product of two has at most 6 significant bits,
    so the lifted features are exact in bf16."""
    return rng.integers(-7, 8, size=shape).astype(np.float64) / (1 << bits)


# ---------------------------------------------------------------------------- rounding
def test_round_bf16_exact_values_unchanged():
    x = np.array([0.0, 1.0, -0.5, 3.0, 1.0 + 2.0 ** -7, -(1.0 + 2.0 ** -7), 2.0 ** -20, 96.0])
    assert np.array_equal(psd_lift.round_bf16_rne(x), x)


def test_round_bf16_hand_values():
    a = 1.0 + 2.0 ** -7                       # bf16-exact
    # a*a = 1 + 2^-6 + 2^-14: the dropped part is below half an ulp (2^-8) -> 1 + 2^-6
    assert psd_lift.round_bf16_rne(a * a) == 1.0 + 2.0 ** -6
    # a*1.5 = 1.5 + 1.5 ulp (ulp 2^-7 in [1, 2)): a tie between 1.5+1ulp (odd) and 1.5+2ulp
    # (even) -> 1.515625
    assert a * 1.5 == 1.51171875
    assert psd_lift.round_bf16_rne(a * 1.5) == 1.515625
    # 1.25 * 1.203125 = 1.50390625 = 1.5 + 0.5 ulp: a tie between 1.5 (even) and 1.5078125
    # (odd) -> 1.5, and the same with the sign flipped
    assert 1.25 * 1.203125 == 1.50390625
    assert psd_lift.round_bf16_rne(1.25 * 1.203125) == 1.5
    assert psd_lift.round_bf16_rne(-1.25 * 1.203125) == -1.5
    # just above that tie rounds up
    assert psd_lift.round_bf16_rne(1.50390625 + 2.0 ** -20) == 1.5078125


# ---------------------------------------------------------------------------- the lift
def test_lift_identities_on_exact_features():
    rng = np.random.default_rng(7)
    u = _dyadic(rng, (50, P))
    w = _dyadic(rng, (50, P))
    fu, fw = psd_lift.psd_features(u), psd_lift.psd_features(w)
    assert fu.shape == (50, P * P)
    assert np.array_equal(np.sum(fu * fw, axis=-1), np.sum(u * w, axis=-1) ** 2)
    assert np.array_equal(np.sum(fu * fu, axis=-1), np.sum(u * u, axis=-1) ** 2)


def test_lift_closed_form_two_hot():
    a, b = 3, 11
    u = np.zeros(P)
    u[a], u[b] = 1.0, -2.0
    f = psd_lift.psd_features(u)
    expect = np.zeros(P * P)
    expect[a * P + a] = 1.0
    expect[a * P + b] = expect[b * P + a] = -2.0
    expect[b * P + b] = 4.0
    assert np.array_equal(f, expect)


def test_lift_rounds_each_feature():
    u = np.zeros(P)
    u[0], u[1] = 1.0 + 2.0 ** -7, 1.5
    u[2], u[3] = 1.25, 1.203125
    f = psd_lift.psd_features(u)
    assert f[0 * P + 1] == 1.515625 and f[1 * P + 0] == 1.515625   # the tie that rounds up
    assert f[2 * P + 3] == 1.5 and f[3 * P + 2] == 1.5             # the tie that rounds down
    assert f[0] == 1.0 + 2.0 ** -6                                   # below half an ulp
    assert f[1 * P + 1] == 2.25


# ---------------------------------------------------------------------------- forward
def _orthonormal_case(rng, T=12, H=2, dv=5):
    """One-hot u_k with a distinct index per token (psi(e_a) = e_{aP+a}: orthonormal keys)."""
    uq = _dyadic(rng, (1, T, H, P))
    uk = np.zeros((1, T, H, P))
    for h in range(H):
        idx = rng.permutation(P)[:T]
        uk[0, np.arange(T), h, idx] = 1.0
    v = rng.standard_normal((1, T, H, dv))
    la = np.log(rng.uniform(0.6, 1.0, (1, T, H)))
    eta = rng.uniform(0.1, 1.0, (1, T, H))
    return uq, uk, v, la, eta


def test_forward_orthonormal_lifted_keys_closed_form():
    rng = np.random.default_rng(3)
    uq, uk, v, la, eta = _orthonormal_case(rng)
    eps = 0.25
    o, _ = psd_lift.forward_psd(uq, uk, v, la, eta, eps)
    T, H = uq.shape[1], uq.shape[2]
    beta = eta / (1.0 + np.float64(np.float32(eps)))   # ||psi(e_a)||^2 = 1
    g = np.cumsum(la, axis=1)
    for h in range(H):
        qk = (uq[0, :, h, :] @ uk[0, :, h, :].T) ** 2    # psi(u_q).psi(u_k) = (u_q.u_k)^2
        M = np.tril(np.exp(g[0, :, h][:, None] - g[0, :, h][None, :]))
        expect = (qk * M) @ (beta[0, :, h][:, None] * v[0, :, h, :])
        np.testing.assert_allclose(o[0, :, h, :], expect, rtol=1e-12, atol=1e-12)


def test_forward_full_step_self_readout():
    """u_q = u_k with eta = 1, eps = 0: every output is the token's own value."""
    rng = np.random.default_rng(5)
    T, H, dv = 24, 2, 6
    u = rng.standard_normal((1, T, H, P))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    u = psd_lift.round_bf16_rne(u)
    v = rng.standard_normal((1, T, H, dv))
    la = np.log(rng.uniform(0.5, 1.0, (1, T, H)))
    o, _ = psd_lift.forward_psd(u, u, v, la, np.ones((1, T, H)), 0.0)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-10)


# ---------------------------------------------------------------------------- mutants
def _mutant_features(kind):
    real = psd_lift.psd_features

    def f(u):
        u = np.asarray(u, dtype=np.float64)
        outer = u[..., :, None] * u[..., None, :]
        if kind == "diagonal_only":
            outer = outer * np.eye(u.shape[-1])
        elif kind == "abs_factor":
            outer = u[..., :, None] * np.abs(u)[..., None, :]
        flat = outer.reshape(*u.shape[:-1], -1)
        if kind == "no_rounding":
            return flat
        if kind == "truncation":
            bits = flat.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
            return bits.view(np.float32).astype(np.float64)
        if kind == "half_up":
            bits = (flat.astype(np.float32).view(np.uint32).astype(np.uint64) + np.uint64(0x8000)) \
                & np.uint64(0xFFFF0000)
            return bits.astype(np.uint32).view(np.float32).astype(np.float64)
        return real(u) if kind == "none" else psd_lift.round_bf16_rne(flat)
    return f


PIN_TESTS = [
    test_lift_identities_on_exact_features,
    test_lift_closed_form_two_hot,
    test_lift_rounds_each_feature,
    test_forward_orthonormal_lifted_keys_closed_form,
    test_forward_full_step_self_readout,
]


@pytest.mark.parametrize("kind", ["diagonal_only", "abs_factor", "no_rounding", "truncation", "half_up"])
def test_pins_catch_feature_mutant(kind, monkeypatch):
    monkeypatch.setattr(psd_lift, "psd_features", _mutant_features(kind))
    caught = 0
    for t in PIN_TESTS:
        try:
            t()
        except AssertionError:
            caught += 1
    assert caught > 0, f"mutant {kind} passed every pin"


def test_pins_catch_query_lifted_from_keys(monkeypatch):
    def wrong(uq, uk, v, la, eta, eps, init_state=None, beta_mode="kaczmarz"):
        f = psd_lift.psd_features(uk)
        return kla_ref.forward(f, f, v, la, eta, eps, init_state, beta_mode)
    monkeypatch.setattr(psd_lift, "forward_psd", wrong)
    with pytest.raises(AssertionError):
        test_forward_orthonormal_lifted_keys_closed_form()


def test_unmutated_passes_every_pin(monkeypatch):
    monkeypatch.setattr(psd_lift, "psd_features", _mutant_features("none"))
    for t in PIN_TESTS:
        t()
