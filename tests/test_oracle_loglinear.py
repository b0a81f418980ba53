"""Pins of the log-linear KLA oracle (oracle/loglinear.py) against what the pages and the
mathematics fix, and planted mistakes that the pins must catch (CPU only).

  levels           hand-derived Fenwick buckets for small positions, and bucket sizes:
                   level l >= 1 holds 2^(l-1) tokens exactly when bit l-1 of t is set
                   (Log-Linear page: exponentially growing buckets, recent tokens finest)
  lambda = 1       the buckets sum to the KLA state: both forms equal the KLA oracle
  one-hot level 0  only the token's own write is read: o_t = beta_t (q_t . k_t) v_t
  orthonormal      with orthonormal keys the delta rule drops out and the definition is the
                   page's parallel form O = (Q K^T . M_H) V, M_H[t,s] = lambda_t^(l(t,s)) e^{g_t-g_s}
  two forms        the recurrent form (bucket merges) equals the token-pair definition
"""
import numpy as np
import pytest
from scipy.linalg import hadamard

from oracle import kla_ref, loglinear


def _inputs(rng, B, T, H, dk, dv, L, knorm=True):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if knorm:
        k *= np.exp(0.5 * rng.standard_normal((B, T, H, 1)))
    v = rng.standard_normal((B, T, H, dv))
    la = np.log(rng.uniform(0.6, 1.0, (B, T, H)))
    eta = rng.uniform(0.1, 1.0, (B, T, H))
    lam = rng.uniform(0.2, 1.5, (B, T, H, L))
    return q, k, v, la, eta, lam


def _recurrent(q, k, v, la, eta, lam, eps, beta_mode="kaczmarz"):
    """Run the recurrent form from empty buckets; returns outputs [B, T, H, dv] and the
    bucket states after the last token."""
    B, T, H, dk = q.shape
    dv, L = v.shape[-1], lam.shape[-1]
    S = np.zeros((B, H, L, dk, dv))
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        o[:, t], S = loglinear.decode_step_loglinear(S, t, q[:, t], k[:, t], v[:, t], la[:, t], eta[:, t],
                                                     lam[:, t], eps, beta_mode)
    return o, S


# ---------------------------------------------------------------------------- levels
def test_levels_hand_derived():
    # t = 3 (0b11): s = 2 differs in bit 0 -> 1; s = 1, 0 differ in bit 1 -> 2
    assert [loglinear.level(3, s) for s in range(4)] == [2, 2, 1, 0]
    # t = 4 (0b100): every earlier token differs in bit 2 -> 3
    assert [loglinear.level(4, s) for s in range(5)] == [3, 3, 3, 3, 0]
    # t = 6 (0b110): s = 5, 4 differ in bit 1 -> 2; s = 0..3 differ in bit 2 -> 3
    assert [loglinear.level(6, s) for s in range(7)] == [3, 3, 3, 3, 2, 2, 0]
    # t = 7 (0b111)
    assert [loglinear.level(7, s) for s in range(8)] == [3, 3, 3, 3, 2, 2, 1, 0]
    assert loglinear.occupied_levels(0) == [0]
    assert loglinear.occupied_levels(6) == [0, 2, 3]


def test_bucket_sizes():
    for t in range(200):
        counts = {}
        for s in range(t + 1):
            counts[loglinear.level(t, s)] = counts.get(loglinear.level(t, s), 0) + 1
        assert counts.pop(0) == 1
        for l, c in counts.items():
            assert (t >> (l - 1)) & 1 and c == 1 << (l - 1)
        assert sorted([0, *counts]) == loglinear.occupied_levels(t)


# ---------------------------------------------------------------------------- reductions
@pytest.mark.parametrize("beta_mode", ["kaczmarz", "direct"])
def test_unit_weights_give_kla(beta_mode):
    rng = np.random.default_rng(1)
    B, T, H, dk, dv, L = 2, 23, 2, 6, 5, 6
    q, k, v, la, eta, _ = _inputs(rng, B, T, H, dk, dv, L, knorm=beta_mode == "kaczmarz")
    lam = np.ones((B, T, H, L))
    o_ref, S_ref = kla_ref.forward(q, k, v, la, eta, 1e-6, beta_mode=beta_mode)
    o1 = loglinear.forward_loglinear(q, k, v, la, eta, lam, 1e-6, beta_mode)
    np.testing.assert_allclose(o1, o_ref, rtol=1e-10, atol=1e-10)
    o2, S = _recurrent(q, k, v, la, eta, lam, 1e-6, beta_mode)
    np.testing.assert_allclose(o2, o_ref, rtol=1e-10, atol=1e-10)
    occ = loglinear.occupied_levels(T - 1)
    np.testing.assert_allclose(S[:, :, occ].sum(axis=2), S_ref, rtol=1e-10, atol=1e-10)


def test_level_zero_only_reads_own_write():
    rng = np.random.default_rng(2)
    B, T, H, dk, dv, L = 1, 19, 3, 5, 4, 6
    q, k, v, la, eta, lam = _inputs(rng, B, T, H, dk, dv, L)
    lam[..., 1:] = 0.0
    beta = kla_ref.kaczmarz_beta(k, eta, 1e-6)
    expect = (lam[..., 0] * beta * np.sum(q * k, axis=-1))[..., None] * v
    np.testing.assert_allclose(loglinear.forward_loglinear(q, k, v, la, eta, lam, 1e-6), expect, rtol=1e-12,
                               atol=1e-12)
    np.testing.assert_allclose(_recurrent(q, k, v, la, eta, lam, 1e-6)[0], expect, rtol=1e-12, atol=1e-12)


def test_orthonormal_keys_give_hierarchical_parallel_form():
    rng = np.random.default_rng(3)
    dk, T, dv, L = 16, 16, 3, 5
    Hd = hadamard(dk) / np.sqrt(dk)
    q = rng.standard_normal((1, T, 1, dk))
    k = Hd[rng.permutation(dk)[:T]][None, :, None, :] * rng.uniform(0.5, 2.0, (1, T, 1, 1))
    v = rng.standard_normal((1, T, 1, dv))
    la = np.log(rng.uniform(0.5, 1.0, (1, T, 1)))
    eta = rng.uniform(0.1, 1.0, (1, T, 1))
    lam = rng.uniform(0.2, 1.5, (1, T, 1, L))
    beta = kla_ref.kaczmarz_beta(k, eta, 1e-6)[0, :, 0]
    g = np.cumsum(la[0, :, 0])
    M = np.zeros((T, T))
    for t in range(T):
        for s in range(t + 1):
            M[t, s] = lam[0, t, 0, loglinear.level(t, s)] * np.exp(g[t] - g[s])
    QK = q[0, :, 0] @ k[0, :, 0].T
    expect = (QK * M) @ (beta[:, None] * v[0, :, 0])
    np.testing.assert_allclose(loglinear.forward_loglinear(q, k, v, la, eta, lam, 1e-6)[0, :, 0], expect,
                               rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(_recurrent(q, k, v, la, eta, lam, 1e-6)[0][0, :, 0], expect, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("beta_mode", ["kaczmarz", "direct"])
def test_recurrent_form_equals_definition(beta_mode):
    rng = np.random.default_rng(4)
    B, T, H, dk, dv, L = 2, 37, 2, 7, 5, 7
    q, k, v, la, eta, lam = _inputs(rng, B, T, H, dk, dv, L, knorm=beta_mode == "kaczmarz")
    o1 = loglinear.forward_loglinear(q, k, v, la, eta, lam, 1e-6, beta_mode)
    o2, _ = _recurrent(q, k, v, la, eta, lam, 1e-6, beta_mode)
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-10)


def test_position_range_is_checked():
    S = np.zeros((1, 1, 3, 2, 2))
    z = np.zeros((1, 1, 2))
    with pytest.raises(ValueError):
        loglinear.decode_step_loglinear(S, 4, z, z, z, np.zeros((1, 1)), np.zeros((1, 1)), np.ones((1, 1, 3)), 1e-6)


# ---------------------------------------------------------------------------- mutants
PINS = [test_levels_hand_derived, test_bucket_sizes, test_level_zero_only_reads_own_write,
        test_orthonormal_keys_give_hierarchical_parallel_form]


def _caught(pins):
    n = 0
    for p in pins:
        try:
            p()
        except AssertionError:
            n += 1
    return n


@pytest.mark.parametrize("kind", ["msb_without_plus_one", "lowest_differing_bit", "distance_log"])
def test_pins_catch_level_mutant(kind, monkeypatch):
    def bad(t, s):
        if s == t:
            return 0
        if kind == "msb_without_plus_one":
            return int(t ^ s).bit_length() - 1
        if kind == "lowest_differing_bit":
            x = t ^ s
            return (x & -x).bit_length()
        return int(t - s).bit_length()
    monkeypatch.setattr(loglinear, "level", bad)
    assert _caught(PINS) > 0


@pytest.mark.parametrize("kind", ["merge_one_level_low", "no_transition_on_old_buckets", "lambda_of_source"])
def test_pins_catch_recurrent_mutant(kind, monkeypatch):
    real = loglinear.decode_step_loglinear

    def bad(states, t, q, k, v, log_alpha, eta, lam, eps, beta_mode="kaczmarz"):
        S = np.array(states, dtype=np.float64)
        alpha = np.exp(np.asarray(log_alpha, dtype=np.float64))
        beta = kla_ref.write_strength(k, eta, eps, beta_mode)
        new = np.zeros_like(S)
        if t > 0:
            j = (t & -t).bit_length() - 1
            for l in loglinear.occupied_levels(t - 1):
                Sl = S[:, :, l]
                if kind != "no_transition_on_old_buckets" or l == 0:
                    kS = np.einsum("nhk,nhkv->nhv", k, Sl)
                    Sl = alpha[..., None, None] * (Sl - beta[..., None, None] * k[..., :, None] * kS[..., None, :])
                dest = (j if kind == "merge_one_level_low" else j + 1) if l <= j else l
                new[:, :, dest] += Sl
        new[:, :, 0] = new[:, :, 0] * 0 + beta[..., None, None] * k[..., :, None] * v[..., None, :]
        o = np.zeros(np.shape(v))
        for l in loglinear.occupied_levels(t):
            w = lam[:, :, l] if kind != "lambda_of_source" else lam[:, :, min(l + 1, lam.shape[2] - 1)]
            o += w[..., None] * np.einsum("nhkv,nhk->nhv", new[:, :, l], q)
        return o, new

    monkeypatch.setattr(loglinear, "decode_step_loglinear", bad)
    with pytest.raises(AssertionError):
        test_recurrent_form_equals_definition("kaczmarz")
    monkeypatch.setattr(loglinear, "decode_step_loglinear", real)
