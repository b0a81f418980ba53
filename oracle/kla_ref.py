"""CPU oracle for the KLA forward recurrence, in float64 (NumPy).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything under
``oracle/``. The library in ``delta_rule_recurrence_kla_amd`` never does, and
this code shares nothing with it.

What it computes is the plain token-by-token definition of the write, from the
Kaczmarz Linear Attention (KLA) page:

  * section "Theoretical derivation": the write finds the state nearest to the
    decayed previous state that satisfies S^T k_t = v_t;
  * section "KLA update rule": beta_t = eta_t / (||k_t||^2 + eps),
    S_t = S~ + beta_t k_t e_t^T with residual e_t = v_t - S~^T k_t;
  * section "Implementation": the decay gate of Gated DeltaNet is kept.

Readings where the page is silent (each also listed in the design doc):
  * S~ = alpha_t * S_{t-1} with alpha_t = exp(log_alpha_t): the current token's
    decay is applied before the current token's write;
  * the readout is o_t = S_t^T q_t, taken after the write, with no 1/sqrt(dk);
  * eps is the float32 value the kernels receive;
  * if ||k_t||^2 + eps == 0 the write is skipped (beta_t = 0).

A second write-strength mode, beta_mode="direct", is the Gated DeltaNet baseline that
the same page sets KLA against (section "Problem statement"): a learned scalar used as the
step size as it is, with no division by ||k_t||^2 + eps. The learned scalar arrives in the
same ``eta`` input. Everything else in the recurrence is unchanged.

Every pin in tests/test_oracle_pins.py exercises this file; none is "parity
unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = ["kaczmarz_beta", "write_strength", "step", "forward", "decode_step"]

BETA_MODES = ("kaczmarz", "direct")


def kaczmarz_beta(k_t: np.ndarray, eta_t, eps) -> np.ndarray:
    """beta_t = eta_t / (||k_t||^2 + eps)  (KLA page, "KLA update rule", the beta_t equation).

    ``k_t`` has the key on its last axis; returns one beta per leading index.
    A zero denominator (only reachable with eps = 0 and k_t = 0) gives beta = 0.
    """
    k_t = np.asarray(k_t, dtype=np.float64)
    denom = np.sum(k_t * k_t, axis=-1) + np.float64(np.float32(eps))
    eta_t = np.asarray(eta_t, dtype=np.float64)
    safe = np.where(denom != 0.0, denom, 1.0)
    return np.where(denom != 0.0, eta_t / safe, 0.0)


def write_strength(k_t, eta_t, eps, beta_mode="kaczmarz") -> np.ndarray:
    """beta_t of the write: the Kaczmarz step (KLA page, "KLA update rule") or, in the
    "direct" mode, the learned scalar eta_t itself (the Gated DeltaNet rule of the
    page's "Problem statement")."""
    if beta_mode == "kaczmarz":
        return kaczmarz_beta(k_t, eta_t, eps)
    if beta_mode == "direct":
        k_t = np.asarray(k_t, dtype=np.float64)
        return np.broadcast_to(np.asarray(eta_t, dtype=np.float64), k_t.shape[:-1]).copy()
    raise ValueError(f"beta_mode must be one of {BETA_MODES}")


def step(S, q_t, k_t, v_t, log_alpha_t, eta_t, eps, beta_mode="kaczmarz"):
    """One token of the recurrence for any number of independent heads.

    S: [..., dk, dv] state before the token; q_t, k_t: [..., dk]; v_t: [..., dv];
    log_alpha_t, eta_t: [...]. Returns (o_t [..., dv], S_t [..., dk, dv]) in float64.
    """
    S = np.asarray(S, dtype=np.float64)
    q_t = np.asarray(q_t, dtype=np.float64)
    k_t = np.asarray(k_t, dtype=np.float64)
    v_t = np.asarray(v_t, dtype=np.float64)
    alpha = np.exp(np.asarray(log_alpha_t, dtype=np.float64))
    beta = write_strength(k_t, eta_t, eps, beta_mode)
    S_dec = alpha[..., None, None] * S                      # S~ = alpha_t S_{t-1}
    e = v_t - np.einsum("...kv,...k->...v", S_dec, k_t)     # e_t = v_t - S~^T k_t
    S_new = S_dec + beta[..., None, None] * (k_t[..., :, None] * e[..., None, :])  # S~ + beta k e^T
    o = np.einsum("...kv,...k->...v", S_new, q_t)           # o_t = S_t^T q_t
    return o, S_new


def forward(q, k, v, log_alpha, eta, eps, init_state=None, beta_mode="kaczmarz"):
    """Whole-sequence forward, token by token.

    q, k: [B, T, H, dk]; v: [B, T, H, dv]; log_alpha, eta: [B, T, H];
    init_state: [B, H, dk, dv] or None (zeros). Returns (o [B, T, H, dv], S_T [B, H, dk, dv]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if init_state is None:
        S = np.zeros((B, H, dk, dv), np.float64)
    else:
        S = np.array(init_state, dtype=np.float64)
    o = np.zeros((B, T, H, dv), np.float64)
    for t in range(T):
        o[:, t], S = step(S, q[:, t], k[:, t], v[:, t], log_alpha[:, t], eta[:, t], eps, beta_mode)
    return o, S


def decode_step(state, q, k, v, log_alpha, eta, eps, beta_mode="kaczmarz"):
    """One decode step: the same single-token update for N x H states.

    state: [N, H, dk, dv]; q, k: [N, H, dk]; v: [N, H, dv]; gates [N, H].
    Returns (o [N, H, dv], new_state [N, H, dk, dv]).
    """
    return step(state, q, k, v, log_alpha, eta, eps, beta_mode)
