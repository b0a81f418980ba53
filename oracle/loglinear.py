"""CPU oracle for log-linear KLA, in float64 (NumPy): Fenwick-bucketed states with
per-level output weights.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything under
``oracle/``. The library never does, and this code shares nothing with it.

The Log-Linear page ("Mathematical formalization", recurrent form) keeps one state
S_t^(l) per Fenwick bucket l of the prefix and reads out
    o_t = sum_l lambda_t^(l) q_t^T S_t^(l),
with buckets that grow exponentially with distance (small for recent tokens, large
for old ones); its parallel form is O = (Q K^T . M_H) V with a hierarchical mask M_H.
The page names Log-Linear Gated DeltaNet; here the same construction is put on the KLA
recurrence of kla_ref. Readings where the page is silent (each also listed in
the design doc):
  * bucket of token s as seen from token t (0-based positions, s <= t): level 0 if
    s == t, else the position of the highest bit in which s and t differ, plus one.
    At position t, level l >= 1 then holds the 2^(l-1) tokens below the l-th bit of t
    exactly when that bit of t is set;
  * a bucket's state is the part of the KLA state that its tokens contributed: with
    A_t = alpha_t (I - beta_t k_t k_t^T) (the KLA write in product form, S_t = A_t S_{t-1}
    + beta_t k_t v_t^T), S_t^(l) = sum over s in bucket l of A_t ... A_{s+1} beta_s k_s v_s^T.
    The buckets sum to the KLA state, so lambda = 1 gives back KLA;
  * lambda_t^(l) is an input per token, head and level (data-dependent weights);
  * the recurrence starts from empty buckets (no initial state).

Two independent forms:
  forward_loglinear        the definition token pair by token pair: o_t = sum_{s<=t}
                           lambda_t^(level(t,s)) beta_s (q_t^T A_t...A_{s+1} k_s) v_s
  decode_step_loglinear    the recurrent form: every bucket takes the token's transition,
                           the buckets that the new position joins are summed into one,
                           and the token's own write opens level 0.
"""
from __future__ import annotations

import numpy as np

from . import kla_ref

__all__ = ["level", "forward_loglinear", "decode_step_loglinear", "occupied_levels"]


def level(t: int, s: int) -> int:
    """Fenwick bucket of token s as seen from token t (s <= t): 0 if s == t, else the index
    of the highest bit where the two positions differ, plus one."""
    if s > t:
        raise ValueError("s must not exceed t")
    return 0 if s == t else int(t ^ s).bit_length()


def occupied_levels(t: int):
    """Levels that hold tokens at position t: 0 and l >= 1 whose bit l-1 of t is set."""
    return [0] + [b + 1 for b in range(max(t, 1).bit_length()) if (t >> b) & 1]


def forward_loglinear(q, k, v, log_alpha, eta, lam, eps, beta_mode="kaczmarz"):
    """Whole-sequence log-linear KLA from empty buckets, by token pairs.

    q, k: [B, T, H, dk]; v: [B, T, H, dv]; log_alpha, eta: [B, T, H]; lam: [B, T, H, L].
    Returns o [B, T, H, dv] in float64. Needs T <= 2^(L-1).
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    la = np.asarray(log_alpha, dtype=np.float64)
    lam = np.asarray(lam, dtype=np.float64)
    B, T, H, dk = q.shape
    L = lam.shape[-1]
    if T > (1 << (L - 1)):
        raise ValueError("T exceeds the levels given")
    beta = kla_ref.write_strength(k, eta, eps, beta_mode)          # [B, T, H]
    alpha = np.exp(la)
    o = np.zeros(v.shape, np.float64)
    for b in range(B):
        for h in range(H):
            for t in range(T):
                y = q[b, t, h].copy()                              # y_s = (A_t ... A_{s+1})^T q_t
                acc = np.zeros(v.shape[-1])
                for s in range(t, -1, -1):
                    ks = k[b, s, h]
                    w = beta[b, s, h] * np.dot(y, ks)
                    acc += lam[b, t, h, level(t, s)] * w * v[b, s, h]
                    # move to s - 1: A_s is symmetric, so A_s^T y = alpha_s (y - beta_s k_s (k_s . y))
                    y = alpha[b, s, h] * (y - beta[b, s, h] * ks * np.dot(ks, y))
                o[b, t, h] = acc
    return o


def decode_step_loglinear(states, t, q, k, v, log_alpha, eta, lam, eps, beta_mode="kaczmarz"):
    """One token (position t) of the recurrent form for N x H heads.

    states: [N, H, L, dk, dv] bucket states at position t - 1 (slots of empty levels are
    ignored); q, k: [N, H, dk]; v: [N, H, dv]; log_alpha, eta: [N, H]; lam: [N, H, L].
    Returns (o [N, H, dv], states at position t); slots of levels that the merge empties are
    set to zero.
    """
    S = np.array(states, dtype=np.float64)
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    lam = np.asarray(lam, dtype=np.float64)
    L = S.shape[2]
    if not (0 <= t < (1 << (L - 1))):
        raise ValueError("position out of range for L levels")
    alpha = np.exp(np.asarray(log_alpha, dtype=np.float64))
    beta = kla_ref.write_strength(k, eta, eps, beta_mode)
    new = np.zeros_like(S)
    if t > 0:
        j = (t & -t).bit_length() - 1                # trailing zeros of t
        for l in occupied_levels(t - 1):
            Sl = S[:, :, l]
            # the token's transition on this bucket: A_t S = alpha (S - beta k (k^T S))
            kS = np.einsum("nhk,nhkv->nhv", k, Sl)
            Sl = alpha[..., None, None] * (Sl - beta[..., None, None] * k[..., :, None] * kS[..., None, :])
            dest = j + 1 if l <= j else l            # buckets 0..j join one bucket at level j+1
            new[:, :, dest] += Sl
    new[:, :, 0] = beta[..., None, None] * k[..., :, None] * v[..., None, :]
    o = np.zeros(v.shape, np.float64)
    for l in occupied_levels(t):
        o += lam[:, :, l][..., None] * np.einsum("nhkv,nhk->nhv", new[:, :, l], q)
    return o, new
