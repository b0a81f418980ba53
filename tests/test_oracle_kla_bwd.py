"""Pins of the gradient oracle (oracle/kla_bwd.py), CPU only.

  finite differences   central differences of the forward oracle (kla_ref, a separate code
                       path) for every input element, the start state, both write strengths
  one token            hand-derived gradients of o = eta (k.q) / (||k||^2 + eps) v from a zero state,
                       and of the start state through alpha (I - beta k k^T)
  mutants              plausible slips in the reverse pass (the step size's dependence on ||k||
                       dropped, the decay left out of dS_{t-1}, a sign flipped, the readout taken
                       from the state before the write) each fail the finite-difference pin
"""
import numpy as np
import pytest

from oracle import kla_bwd, kla_ref


def _case(rng, T=7, dk=3, dv=2, direct=False):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    if direct:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, dv))
    la = np.log(rng.uniform(0.5, 1.0, T))
    eta = rng.uniform(0.2, 0.9, T)
    S0 = 0.3 * rng.standard_normal((dk, dv))
    Wo = rng.standard_normal((T, dv))
    WS = rng.standard_normal((dk, dv))
    return q, k, v, la, eta, S0, Wo, WS


def _loss(q, k, v, la, eta, S0, Wo, WS, eps, mode):
    o, S = kla_ref.forward(q[None, :, None], k[None, :, None], v[None, :, None], la[None, :, None],
                           eta[None, :, None], eps, S0[None, None], beta_mode=mode)
    return float(np.sum(Wo * o[0, :, 0]) + np.sum(WS * S[0, 0]))


def _fd(args, idx, eps, mode, h=1e-6):
    """Central difference of the loss in every element of argument number idx."""
    base = [np.array(a, dtype=np.float64) for a in args]
    x = base[idx]
    g = np.zeros_like(x)
    for j in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[j] += h
        xm[j] -= h
        ap, am = list(base), list(base)
        ap[idx], am[idx] = xp, xm
        g[j] = (_loss(*ap, eps, mode) - _loss(*am, eps, mode)) / (2 * h)
    return g


NAMES = ["dq", "dk", "dv", "dlog_alpha", "deta", "dS0"]


def _check_fd(bwd, mode, seed):
    rng = np.random.default_rng(seed)
    q, k, v, la, eta, S0, Wo, WS = _case(rng, direct=mode == "direct")
    eps = 1e-3
    g = bwd(q, k, v, la, eta, eps, Wo, WS, S0, mode)
    args = (q, k, v, la, eta, S0, Wo, WS)
    for name, idx in zip(NAMES, [0, 1, 2, 3, 4, 5]):
        np.testing.assert_allclose(g[name], _fd(args, idx, eps, mode), rtol=1e-5, atol=1e-7, err_msg=name)


def _oracle(q, k, v, la, eta, eps, dO, dS_T, S0, mode):
    return kla_bwd.backward(q, k, v, la, eta, eps, dO, dS_T, S0, mode)


@pytest.mark.parametrize("mode", ["kaczmarz", "direct"])
@pytest.mark.parametrize("seed", [0, 1])
def test_gradients_match_finite_differences(mode, seed):
    _check_fd(_oracle, mode, seed)


def test_one_token_closed_form():
    rng = np.random.default_rng(3)
    dk, dv = 4, 3
    q, k, v = rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv)
    la, eta, eps = -0.2, 0.7, 1e-3
    w = rng.standard_normal(dv)
    g = kla_bwd.backward(q[None], k[None], v[None], np.array([la]), np.array([eta]), eps, w[None])
    d = k @ k + np.float64(np.float32(eps))
    kq, vw = k @ q, v @ w
    np.testing.assert_allclose(g["dv"][0], eta * kq / d * w, rtol=1e-12)
    np.testing.assert_allclose(g["dq"][0], eta / d * vw * k, rtol=1e-12)
    np.testing.assert_allclose(g["dk"][0], eta * vw * (q / d - 2 * kq * k / d ** 2), rtol=1e-12)
    np.testing.assert_allclose(g["deta"][0], kq / d * vw, rtol=1e-12)
    # o = S_1^T q with S_1 = alpha (I - beta k k^T) S_0 + beta k v^T: the start state's gradient is
    # alpha (I - beta k k^T) q w^T, and with S_0 = 0 the decay has none
    alpha, beta = np.exp(la), eta / d
    np.testing.assert_allclose(g["dS0"], alpha * np.outer((np.eye(dk) - beta * np.outer(k, k)) @ q, w), rtol=1e-12)
    assert g["dlog_alpha"][0] == 0.0


# ---------------------------------------------------------------------------- mutants
def _mutant(variant):
    def bwd(q, k, v, la, eta, eps, dO, dS_T, S0, mode):
        _, states = kla_bwd.forward_states(q, k, v, la, eta, eps, S0, mode)
        T, dk = q.shape
        eps64 = np.float64(np.float32(eps))
        dS = np.array(dS_T, dtype=np.float64)
        g = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dlog_alpha", la), ("deta", eta))}
        for t in range(T - 1, -1, -1):
            S_prev, S_t = states[t], states[t + 1]
            a = np.exp(la[t])
            denom = k[t] @ k[t] + eps64
            beta = eta[t] if mode == "direct" else eta[t] / denom
            S_dec = a * S_prev
            e = v[t] - S_dec.T @ k[t]
            g["dq"][t] = (S_prev if variant == "readout_before_write" else S_t) @ dO[t]
            dS = dS + np.outer(q[t], dO[t])
            dS_dec = dS.copy()
            dbeta = k[t] @ dS @ e
            dk_t = beta * (dS @ e)
            de = beta * (dS.T @ k[t])
            g["dv"][t] = de
            dS_dec -= np.outer(k[t], de)
            dk_t += (S_dec @ de) if variant == "residual_sign" else -(S_dec @ de)
            g["dlog_alpha"][t] = a * np.sum(dS_dec * S_prev)
            dS = dS_dec if variant == "no_decay_in_carry" else a * dS_dec
            if mode == "direct":
                g["deta"][t] = dbeta
            else:
                g["deta"][t] = dbeta / denom
                if variant != "beta_constant_in_k":
                    dk_t += 2.0 * k[t] * (-dbeta * eta[t] / denom ** 2)
            g["dk"][t] = dk_t
        g["dS0"] = dS
        return g
    return bwd


@pytest.mark.parametrize("variant", ["beta_constant_in_k", "no_decay_in_carry", "residual_sign",
                                     "readout_before_write"])
def test_finite_differences_catch_mutant(variant):
    with pytest.raises(AssertionError):
        _check_fd(_mutant(variant), "kaczmarz", 0)


def test_unmutated_reimplementation_passes():
    _check_fd(_mutant("none"), "kaczmarz", 0)
