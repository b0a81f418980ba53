"""CPU oracle for the gradients of the KLA forward recurrence, in float64 (NumPy).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything under
``oracle/``. The library never does, and this code shares nothing with it.

Reverse mode through the token loop of kla_ref (KLA page, "KLA update rule": beta_t =
eta_t / (||k_t||^2 + eps), S~ = alpha_t S_{t-1}, e_t = v_t - S~^T k_t,
S_t = S~ + beta_t k_t e_t^T, o_t = S_t^T q_t), for a loss whose gradients with respect
to the outputs (dO) and to the end state (dS_T) are given. Working backwards from
dS = dS_T, each token t takes, in this order:

  o_t = S_t^T q_t            dq_t = S_t do_t;              dS += q_t do_t^T
  S_t = S~ + beta k e^T      dS~ = dS;  dbeta = k^T dS e;  dk = beta dS e;  de = beta dS^T k
  e = v - S~^T k             dv = de;   dS~ -= k de^T;     dk -= S~ de
  S~ = alpha S_{t-1}         dalpha = <dS~, S_{t-1}>;      dS_{t-1} = alpha dS~
  alpha = exp(log_alpha)     dlog_alpha = alpha dalpha
  beta = eta / (n + eps)     deta = dbeta / (n + eps);     dk += 2 k (-dbeta eta / (n + eps)^2)
                             (direct mode: deta = dbeta; a zero denominator gives beta = 0 and
                             no gradient through it)

The states S_{t-1} and S_t come from a forward pass that keeps every state.
"""
from __future__ import annotations

import numpy as np

from . import kla_ref

__all__ = ["forward_states", "backward"]


def forward_states(q, k, v, log_alpha, eta, eps, init_state=None, beta_mode="kaczmarz"):
    """Token loop of kla_ref for one sequence of one head, keeping every state.

    q, k: [T, dk]; v: [T, dv]; log_alpha, eta: [T]; init_state: [dk, dv] or None.
    Returns (o [T, dv], states [T + 1, dk, dv]) with states[0] the start state.
    """
    T, dk = np.shape(q)
    dv = np.shape(v)[-1]
    S = np.zeros((dk, dv)) if init_state is None else np.array(init_state, dtype=np.float64)
    states = [S]
    o = np.zeros((T, dv))
    for t in range(T):
        o[t], S = kla_ref.step(S, q[t], k[t], v[t], log_alpha[t], eta[t], eps, beta_mode)
        states.append(S)
    return o, np.stack(states)


def backward(q, k, v, log_alpha, eta, eps, dO, dS_T=None, init_state=None, beta_mode="kaczmarz"):
    """Gradients of a loss with d loss / d o = dO [T, dv] and d loss / d S_T = dS_T [dk, dv]
    (None: zero) for one sequence of one head.

    Returns a dict with dq, dk [T, dk], dv [T, dv], dlog_alpha, deta [T], dS0 [dk, dv].
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    la = np.asarray(log_alpha, dtype=np.float64)
    et = np.asarray(eta, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    T, dk = q.shape
    dv = v.shape[-1]
    _, states = forward_states(q, k, v, la, et, eps, init_state, beta_mode)
    eps64 = np.float64(np.float32(eps))
    dS = np.zeros((dk, dv)) if dS_T is None else np.array(dS_T, dtype=np.float64)
    g = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dlog_alpha", la), ("deta", et))}
    for t in range(T - 1, -1, -1):
        S_prev, S_t = states[t], states[t + 1]
        a = np.exp(la[t])
        n = float(k[t] @ k[t])
        denom = n + eps64
        if beta_mode == "direct":
            beta = et[t]
        else:
            beta = et[t] / denom if denom != 0.0 else 0.0
        S_dec = a * S_prev
        e = v[t] - S_dec.T @ k[t]
        # o_t = S_t^T q_t
        g["dq"][t] = S_t @ dO[t]
        dS = dS + np.outer(q[t], dO[t])
        # S_t = S~ + beta k e^T
        dS_dec = dS.copy()
        dbeta = float(k[t] @ dS @ e)
        dk_t = beta * (dS @ e)
        de = beta * (dS.T @ k[t])
        # e = v - S~^T k
        g["dv"][t] = de
        dS_dec -= np.outer(k[t], de)
        dk_t -= S_dec @ de
        # S~ = alpha S_{t-1}
        dalpha = float(np.sum(dS_dec * S_prev))
        g["dlog_alpha"][t] = a * dalpha
        dS = a * dS_dec
        # beta
        if beta_mode == "direct":
            g["deta"][t] = dbeta
        elif denom != 0.0:
            g["deta"][t] = dbeta / denom
            dk_t += 2.0 * k[t] * (-dbeta * et[t] / denom ** 2)
        g["dk"][t] = dk_t
    g["dS0"] = dS
    return g
