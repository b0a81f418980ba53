"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test runs on both oracle builds (NumPy and C). Every pin is chosen so that
a plausible slip in the oracle (a dropped term, a wrong sign, a transposed
operand, the decay or the readout in the wrong place) fails at least one:

  worked example   hand-derived exact fractions (tests/golden)           whole step, readout time, transposes
  constraint       eta=1, eps=0: S_t^T k_t = v_t                         beta's norm, residual sign, decay placement
  min-norm         change equals pinv-based minimum-norm correction     projection (KLA "Theoretical derivation")
  line search      beta minimises the per-token loss along k e^T         (KLA "Key properties" 2)
  normalised SGD   change = -beta * finite-difference gradient           (KLA "Key properties" 3)
  orthogonal keys  delta rule reduces to the masked form (QK^T . M) B V  decay mask, beta, eta, eps, readout
  overwrite        repeated key keeps only the latest value              (KATA "Results", repeated-key overwrite)
  pure decay       eta=0 leaves alpha-products of the initial state
  product form     S_T = A_T..A_1 S_0 + sum_i A_T..A_{i+1} beta_i k_i v_i^T  whole recurrence, other algebra
  linearity        joint linearity in (V, S_0); causality
  NumPy == C       the two builds agree to 1e-12
  direct mode      the learned-scalar step (KLA "Problem statement") equals KLA on unit keys,
                   and the residual law (1 - beta ||k||^2) fixes how each mode scales a write
"""
import os

import numpy as np
import pytest

from oracle import kla_ref, cref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _c_forward(q, k, v, la, eta, eps, init_state=None):
    """C oracle with NumPy oracle's signature and shapes (all heads)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out, fin = cref.forward(q, k, v, la, eta, eps, init_state)
    out = out.reshape(B, H, T, dv).transpose(0, 2, 1, 3)
    return out, fin.reshape(B, H, dk, dv)


IMPLS = {"numpy": kla_ref.forward, "c": _c_forward}


@pytest.fixture(params=sorted(IMPLS))
def fwd(request):
    return IMPLS[request.param]


def _rand(rng, B, T, H, dk, dv, alpha_lo=0.6, eta_range=(0.1, 1.0), knorm=True):
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    if knorm:
        k *= np.exp(0.5 * rng.standard_normal((B, T, H, 1))).astype(np.float32)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    la = np.log(rng.uniform(alpha_lo, 1.0, (B, T, H))).astype(np.float32)
    eta = rng.uniform(*eta_range, (B, T, H)).astype(np.float32)
    return q, k, v, la, eta


# ----------------------------------------------------------------------------
def _read_golden():
    rows, final = [], None
    with open(os.path.join(GOLDEN, "kla_worked_dk2_dv2.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0] == "final":
                final = np.array([float(x) for x in parts[1:]]).reshape(2, 2)
            else:
                rows.append([float(x) for x in parts])
    return np.array(rows), final


def test_worked_example_exact(fwd):
    rows, final = _read_golden()
    T = len(rows)
    k = rows[:, 1:3].reshape(1, T, 1, 2)
    v = rows[:, 3:5].reshape(1, T, 1, 2)
    q = rows[:, 5:7].reshape(1, T, 1, 2)
    la = np.log(rows[:, 7]).reshape(1, T, 1)
    eta = rows[:, 8].reshape(1, T, 1)
    o_exp = rows[:, 9:11]
    o, S = fwd(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32),
               la.astype(np.float32), eta.astype(np.float32), 0.0)
    # log(0.5) in float32 is not exactly log(1/2): allow its rounding (1e-7 relative)
    np.testing.assert_allclose(o[0, :, 0], o_exp, rtol=0, atol=1e-6)
    np.testing.assert_allclose(S[0, 0], final, rtol=0, atol=1e-6)


def test_worked_example_exact_no_decay_rounding():
    """The same example with alpha entered through exp(log alpha) in float64 exactly."""
    rows, final = _read_golden()
    T = len(rows)
    S = np.zeros((2, 2))
    for t in range(T):
        o, S = kla_ref.step(S, rows[t, 5:7], rows[t, 1:3], rows[t, 3:5], np.log(rows[t, 7]), rows[t, 8], 0.0)
        np.testing.assert_allclose(o, rows[t, 9:11], rtol=0, atol=1e-14)
    np.testing.assert_allclose(S, final, rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------
def test_constraint_exact_projection(fwd):
    """eta=1, eps=0: every write lands exactly on S_t^T k_t = v_t (dk != dv catches transposes)."""
    rng = np.random.default_rng(1)
    B, T, H, dk, dv = 2, 12, 2, 7, 5
    q, k, v, la, _ = _rand(rng, B, T, H, dk, dv)
    eta = np.ones((B, T, H), np.float32)
    S0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    for t in range(1, T + 1):
        _, S = fwd(q[:, :t], k[:, :t], v[:, :t], la[:, :t], eta[:, :t], 0.0, S0)
        resid = np.einsum("bhkv,bhk->bhv", S, k[:, t - 1].astype(np.float64)) - v[:, t - 1]
        assert np.max(np.abs(resid)) < 1e-10


def test_minimum_norm_change():
    """The write is the minimum-Frobenius-norm change meeting the constraint
    (KLA "Theoretical derivation"): compare with the pseudo-inverse solution and check
    Pythagoras against random null-space perturbations."""
    rng = np.random.default_rng(2)
    dk, dv = 6, 4
    for _ in range(20):
        S_prev = rng.standard_normal((dk, dv))
        k = rng.standard_normal(dk) * rng.uniform(0.1, 3)
        v = rng.standard_normal(dv)
        q = rng.standard_normal(dk)
        la = np.log(rng.uniform(0.5, 1))
        _, S = kla_ref.step(S_prev, q, k, v, la, 1.0, 0.0)
        S_dec = np.exp(la) * S_prev
        dS = S - S_dec
        # minimum-norm solution of dS^T k = v - S_dec^T k, column by column, via pinv
        e = v - S_dec.T @ k
        dS_pinv = np.linalg.pinv(k[None, :]) @ e[None, :]
        np.testing.assert_allclose(dS, dS_pinv, rtol=1e-12, atol=1e-12)
        # any other feasible change dS + Z (Z^T k = 0) is no smaller: Pythagoras
        Z = rng.standard_normal((dk, dv))
        Z -= np.outer(k, k @ Z) / (k @ k)
        assert np.allclose(Z.T @ k, 0, atol=1e-12)
        lhs = np.sum((dS + Z) ** 2)
        assert abs(lhs - (np.sum(dS ** 2) + np.sum(Z ** 2))) < 1e-10 * max(1.0, lhs)


def test_exact_line_search():
    """With eta=1, eps=0 the step size along k e^T minimises the per-token loss
    (KLA "Key properties", exact line search), found here by a bounded scalar search."""
    from scipy.optimize import minimize_scalar
    rng = np.random.default_rng(3)
    dk, dv = 5, 3
    for _ in range(10):
        S_prev = rng.standard_normal((dk, dv))
        k = rng.standard_normal(dk) * rng.uniform(0.2, 4)
        v = rng.standard_normal(dv)
        _, S = kla_ref.step(S_prev, np.zeros(dk), k, v, 0.0, 1.0, 0.0)
        e = v - S_prev.T @ k
        phi = lambda s: 0.5 * np.sum(((S_prev + s * np.outer(k, e)).T @ k - v) ** 2)
        res = minimize_scalar(phi, bounds=(0, 10 / (k @ k)), method="bounded",
                              options={"xatol": 1e-12})
        # the oracle's effective step: dS = s k e^T
        s_oracle = np.sum((S - S_prev) * np.outer(k, e)) / np.sum(np.outer(k, e) ** 2)
        assert abs(s_oracle - res.x) < 1e-6 * max(1, res.x)
        assert phi(s_oracle) < 1e-20


def test_normalised_sgd_step():
    """The write is S~ - beta * grad_S 0.5||S^T k - v||^2 at S~ (KLA "Key properties",
    normalised SGD), with the gradient taken by central finite differences."""
    rng = np.random.default_rng(4)
    dk, dv = 4, 3
    S_prev = rng.standard_normal((dk, dv))
    k = rng.standard_normal(dk) * 1.7
    v = rng.standard_normal(dv)
    la, eta, eps = np.log(0.8), 0.7, 1e-3
    _, S = kla_ref.step(S_prev, np.zeros(dk), k, v, la, eta, eps)
    S_dec = np.exp(la) * S_prev
    loss = lambda M: 0.5 * np.sum((M.T @ k - v) ** 2)
    grad = np.zeros_like(S_dec)
    h = 1e-6
    for i in range(dk):
        for j in range(dv):
            E = np.zeros_like(S_dec)
            E[i, j] = h
            grad[i, j] = (loss(S_dec + E) - loss(S_dec - E)) / (2 * h)
    beta = eta / (k @ k + np.float32(eps))
    np.testing.assert_allclose(S, S_dec - beta * grad, rtol=1e-7, atol=1e-8)


# ----------------------------------------------------------------------------
def test_orthogonal_keys_reduce_to_masked_form(fwd):
    """With mutually orthogonal keys every residual is v_t itself, so the recurrence
    equals the masked parallel form O = (Q K^T . M) diag(beta) V of linear attention
    (Log-Linear Attention page, "Mathematical formalization", parallel form) with the
    decay mask M[t,i] = prod_{i<j<=t} alpha_j for i <= t (diagonal included)."""
    rng = np.random.default_rng(5)
    B, H, dk, dv, T = 1, 2, 16, 5, 12
    q = rng.standard_normal((B, T, H, dk))
    k = np.zeros((B, T, H, dk))
    from scipy.linalg import hadamard
    # scaled, sign-flipped Hadamard rows: exactly orthogonal even after float32 rounding
    Hd = hadamard(dk).astype(np.float64)
    for h in range(H):
        rows = rng.permutation(dk)[:T]
        signs = rng.choice([-1.0, 1.0], dk)
        k[0, :, h] = Hd[rows] * signs * rng.uniform(0.1, 0.8, (T, 1))
    v = rng.standard_normal((B, T, H, dv))
    la = np.log(rng.uniform(0.5, 1.0, (B, T, H)))
    eta = rng.uniform(0.2, 1.0, (B, T, H))
    eps = 1e-2
    f = lambda a: a.astype(np.float32)
    q, k, v, la, eta = f(q), f(k), f(v), f(la), f(eta)
    o, _ = fwd(q, k, v, la, eta, eps)
    for h in range(H):
        Q, K, V = (x[0, :, h].astype(np.float64) for x in (q, k, v))
        g = np.cumsum(la[0, :, h].astype(np.float64))
        M = np.tril(np.exp(g[:, None] - g[None, :]))
        beta = eta[0, :, h] / (np.sum(K * K, 1) + np.float32(eps))
        O = ((Q @ K.T) * M) @ (beta[:, None] * V)
        np.testing.assert_allclose(o[0, :, h], O, rtol=1e-9, atol=1e-9)


def test_repeated_key_overwrite(fwd):
    """(k, v1) then (k, v2) with eta=1, eps=0, no decay leaves S^T k = v2 and does not
    touch directions orthogonal to k (KATA page, "Results", repeated-key overwrite)."""
    rng = np.random.default_rng(6)
    dk, dv = 8, 3
    k1 = rng.standard_normal(dk)
    kk = np.stack([k1, k1 * 2.5])  # the same address at another scale
    v = rng.standard_normal((2, dv))
    q = rng.standard_normal((2, dk))
    S0 = rng.standard_normal((1, 1, dk, dv))
    f = lambda a: a.astype(np.float32)
    _, S = fwd(f(q[None, :, None]), f(kk[None, :, None]), f(v[None, :, None]),
               np.zeros((1, 2, 1), np.float32), np.ones((1, 2, 1), np.float32), 0.0, f(S0))
    S = S[0, 0]
    kf = f(kk[1]).astype(np.float64)
    np.testing.assert_allclose(S.T @ kf, f(v[1]), atol=1e-10)
    kp = rng.standard_normal(dk)
    k1f = f(kk[0]).astype(np.float64)
    kp -= k1f * (kp @ k1f) / (k1f @ k1f)
    np.testing.assert_allclose(S.T @ kp, f(S0[0, 0]).astype(np.float64).T @ kp, atol=1e-10)


def test_pure_decay(fwd):
    """eta=0: no write, S_t = exp(sum log_alpha) S_0 and o_t = S_t^T q_t."""
    rng = np.random.default_rng(7)
    B, T, H, dk, dv = 1, 9, 3, 6, 4
    q, k, v, la, _ = _rand(rng, B, T, H, dk, dv)
    eta = np.zeros((B, T, H), np.float32)
    S0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    o, S = fwd(q, k, v, la, eta, 1e-6, S0)
    g = np.cumsum(la.astype(np.float64), axis=1)  # [B,T,H]
    for t in range(T):
        St = np.exp(g[:, t])[..., None, None] * S0
        np.testing.assert_allclose(o[:, t], np.einsum("bhkv,bhk->bhv", St, q[:, t]), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S, np.exp(g[:, -1])[..., None, None] * S0, rtol=1e-12)


def test_product_form_brute_force(fwd):
    """Whole recurrence against its closed product form, built from explicit matrices:
    A_i = alpha_i (I - beta_i k_i k_i^T),
    S_t = A_t ... A_1 S_0 + sum_{i<=t} A_t ... A_{i+1} beta_i k_i v_i^T, o_t = S_t^T q_t."""
    rng = np.random.default_rng(8)
    B, T, H, dk, dv = 1, 16, 2, 6, 3
    q, k, v, la, eta = _rand(rng, B, T, H, dk, dv, alpha_lo=0.3, eta_range=(0.0, 1.5))
    eps = 0.05
    S0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    o, S = fwd(q, k, v, la, eta, eps, S0)
    for h in range(H):
        K, V, Q = (x[0, :, h].astype(np.float64) for x in (k, v, q))
        alpha = np.exp(la[0, :, h].astype(np.float64))
        beta = eta[0, :, h].astype(np.float64) / (np.sum(K * K, 1) + np.float64(np.float32(eps)))
        A = [alpha[i] * (np.eye(dk) - beta[i] * np.outer(K[i], K[i])) for i in range(T)]
        for t in range(T):
            # S_t = (A_t...A_0) S0 + sum_i (A_t...A_{i+1}) beta_i k_i v_i^T
            St = np.zeros((dk, dv))
            prod = np.eye(dk)
            for i in range(t, -1, -1):
                St += prod @ (beta[i] * np.outer(K[i], V[i]))
                prod = prod @ A[i]
            St += prod @ S0[0, h].astype(np.float64)
            np.testing.assert_allclose(o[0, t, h], St.T @ Q[t], rtol=1e-10, atol=1e-10)
            if t == T - 1:
                np.testing.assert_allclose(S[0, h], St, rtol=1e-10, atol=1e-10)


def test_linearity_and_causality(fwd):
    """Outputs and final state are jointly linear in (V, S_0) for fixed q, k and gates,
    and changing tokens after t leaves outputs up to t bit-identical."""
    rng = np.random.default_rng(9)
    B, T, H, dk, dv = 1, 20, 2, 5, 4
    q, k, v1, la, eta = _rand(rng, B, T, H, dk, dv)
    # values on a 2^-8 grid and power-of-two weights: a*x + b*y is exact in float32
    grid = lambda x: (np.round(np.clip(x, -4, 4) * 256) / 256).astype(np.float32)
    v1 = grid(v1)
    v2 = grid(rng.standard_normal(v1.shape))
    S1 = grid(rng.standard_normal((B, H, dk, dv)))
    S2 = grid(rng.standard_normal((B, H, dk, dv)))
    a, b = 0.5, -2.0
    o1, F1 = fwd(q, k, v1, la, eta, 1e-6, S1)
    o2, F2 = fwd(q, k, v2, la, eta, 1e-6, S2)
    o3, F3 = fwd(q, k, (a * v1 + b * v2).astype(np.float32), la, eta, 1e-6, (a * S1 + b * S2).astype(np.float32))
    np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(F3, a * F1 + b * F2, rtol=1e-11, atol=1e-11)
    t = 11
    q2, k2, v3 = q.copy(), k.copy(), v1.copy()
    q2[:, t + 1:] += 1
    k2[:, t + 1:] *= 2
    v3[:, t + 1:] -= 3
    o4, _ = fwd(q2, k2, v3, la, eta, 1e-6, S1)
    assert np.array_equal(o4[:, : t + 1], o1[:, : t + 1])
    assert not np.allclose(o4[:, t + 1:], o1[:, t + 1:])


def test_numpy_equals_c():
    rng = np.random.default_rng(10)
    B, T, H, dk, dv = 2, 70, 3, 32, 16
    q, k, v, la, eta = _rand(rng, B, T, H, dk, dv)
    S0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    o1, F1 = kla_ref.forward(q, k, v, la, eta, 1e-6, S0)
    o2, F2 = _c_forward(q, k, v, la, eta, 1e-6, S0)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12 * np.sqrt(np.mean(o1 ** 2)))
    np.testing.assert_allclose(F2, F1, rtol=1e-12, atol=1e-12)
    # head subset: compact outputs equal the full run's slices
    heads = [(1, 2), (0, 0)]
    out, fin = cref.forward(q, k, v, la, eta, 1e-6, S0, heads=heads)
    for n, (b, h) in enumerate(heads):
        np.testing.assert_allclose(out[n], o1[b, :, h], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(fin[n], F1[b, h], rtol=1e-12, atol=1e-12)


def test_decode_step_matches_forward():
    """A decode step is one token of the same recurrence (both oracle builds)."""
    rng = np.random.default_rng(11)
    N, H, dk, dv = 3, 2, 8, 6
    S = rng.standard_normal((N, H, dk, dv)).astype(np.float32)
    q = rng.standard_normal((N, H, dk)).astype(np.float32)
    k = rng.standard_normal((N, H, dk)).astype(np.float32)
    v = rng.standard_normal((N, H, dv)).astype(np.float32)
    la = np.log(rng.uniform(0.5, 1, (N, H))).astype(np.float32)
    eta = rng.uniform(0, 1, (N, H)).astype(np.float32)
    o_ref, S_ref = kla_ref.forward(q[:, None], k[:, None], v[:, None], la[:, None], eta[:, None], 1e-6, S)
    o1, S1 = kla_ref.decode_step(S, q, k, v, la, eta, 1e-6)
    np.testing.assert_allclose(o1, o_ref[:, 0], rtol=1e-14)
    np.testing.assert_allclose(S1, S_ref, rtol=1e-14)
    heads = [(2, 1), (0, 0), (1, 1)]
    st = np.stack([S[a, h] for a, h in heads]).astype(np.float64)
    o2 = cref.decode_step(st, q, k, v, la, eta, 1e-6, heads=heads)
    for n, (a, h) in enumerate(heads):
        np.testing.assert_allclose(o2[n], o1[a, h], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(st[n], S1[a, h], rtol=1e-12, atol=1e-13)


def test_zero_key_zero_eps_skips_write():
    """||k||^2 + eps == 0 (k = 0, eps = 0) is read as no write: beta = 0."""
    S = np.arange(6, dtype=np.float64).reshape(3, 2)
    o, S1 = kla_ref.step(S, np.ones(3), np.zeros(3), np.ones(2), 0.0, 1.0, 0.0)
    np.testing.assert_array_equal(S1, S)


# ----------------------------------------------------------------------------
# The direct write-strength mode: Gated DeltaNet's learned scalar used as the step size as
# given (KLA page, "Problem statement"), beside KLA's beta = eta / (||k||^2 + eps).
def _fwd_mode(impl, mode):
    if impl == "numpy":
        return lambda q, k, v, la, eta, eps, init_state=None: kla_ref.forward(q, k, v, la, eta, eps, init_state,
                                                                                beta_mode=mode)

    def c(q, k, v, la, eta, eps, init_state=None):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        out, fin = cref.forward(q, k, v, la, eta, eps, init_state, beta_mode=mode)
        return out.reshape(B, H, T, dv).transpose(0, 2, 1, 3), fin.reshape(B, H, dk, dv)
    return c


@pytest.mark.parametrize("impl", ["numpy", "c"])
def test_direct_equals_kaczmarz_on_unit_keys(impl):
    """With ||k||^2 + eps = 1 exactly the Kaczmarz step is eta itself, so the modes agree."""
    rng = np.random.default_rng(21)
    B, T, H, dk, dv = 1, 40, 2, 8, 5
    q, _, v, la, eta = _rand(rng, B, T, H, dk, dv)
    k = np.zeros((B, T, H, dk), np.float32)
    for idx in np.ndindex(B, T, H):  # four entries of +-1/2: norm exactly 1 in float32
        k[idx][rng.choice(dk, 4, replace=False)] = rng.choice([-0.5, 0.5], 4)
    a = _fwd_mode(impl, "direct")(q, k, v, la, eta, 0.0)
    b = _fwd_mode(impl, "kaczmarz")(q, k, v, la, eta, 0.0)
    np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-12)
    # and they differ once the keys are not unit vectors
    c_ = _fwd_mode(impl, "direct")(q, 2 * k, v, la, eta, 0.0)
    d_ = _fwd_mode(impl, "kaczmarz")(q, 2 * k, v, la, eta, 0.0)
    assert not np.allclose(c_[1], d_[1])


@pytest.mark.parametrize("impl", ["numpy", "c"])
def test_write_residual_law(impl):
    """A write scales the residual on its own key by (1 - beta ||k||^2): the Kaczmarz step
    leaves 1 - eta whatever the key's norm, while the learned scalar taken as given over-
    corrects a large-norm key (the factor goes below -1) and under-corrects a small one."""
    rng = np.random.default_rng(22)
    dk, dv = 6, 4
    eta32 = np.float32(0.7)
    for scale in (3.0, 0.2):
        S0 = rng.standard_normal((1, 1, dk, dv)).astype(np.float32)
        k = (rng.standard_normal((1, 1, 1, dk)) * scale).astype(np.float32)
        q = rng.standard_normal((1, 1, 1, dk)).astype(np.float32)
        v = rng.standard_normal((1, 1, 1, dv)).astype(np.float32)
        la = np.full((1, 1, 1), np.log(0.9), np.float32)
        eta = np.full((1, 1, 1), eta32, np.float32)
        kk = k[0, 0, 0].astype(np.float64)
        nk = kk @ kk
        S_dec = np.exp(np.float64(la[0, 0, 0])) * S0[0, 0].astype(np.float64)
        e0 = v[0, 0, 0].astype(np.float64) - S_dec.T @ kk
        for mode, factor in (("direct", 1 - np.float64(eta32) * nk), ("kaczmarz", 1 - np.float64(eta32))):
            _, S1 = _fwd_mode(impl, mode)(q, k, v, la, eta, 0.0, S0)
            e1 = v[0, 0, 0].astype(np.float64) - S1[0, 0].T @ kk
            np.testing.assert_allclose(e1, factor * e0, rtol=1e-10, atol=1e-12)
            if mode == "direct":
                assert (factor < -1) if scale > 1 else (factor > 1 - np.float64(eta32))


def test_numpy_equals_c_direct_mode():
    rng = np.random.default_rng(23)
    B, T, H, dk, dv = 2, 50, 2, 16, 8
    q, k, v, la, eta = _rand(rng, B, T, H, dk, dv)
    k *= 0.3  # keep ||k||^2 eta below 2 so the direct write stays stable over the run
    S0 = rng.standard_normal((B, H, dk, dv)).astype(np.float32)
    o1, F1 = kla_ref.forward(q, k, v, la, eta, 1e-6, S0, beta_mode="direct")
    o2, F2 = _fwd_mode("c", "direct")(q, k, v, la, eta, 1e-6, S0)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12 * np.sqrt(np.mean(o1 ** 2)))
    np.testing.assert_allclose(F2, F1, rtol=1e-12, atol=1e-12)
    st = S0.astype(np.float64)[:, :, :, :].reshape(B * H, dk, dv).copy()
    out = cref.decode_step(st, q[:, 0], k[:, 0], v[:, 0], la[:, 0], eta[:, 0], 1e-6, beta_mode="direct")
    o_ref, S_ref = kla_ref.decode_step(S0, q[:, 0], k[:, 0], v[:, 0], la[:, 0], eta[:, 0], 1e-6, beta_mode="direct")
    np.testing.assert_allclose(out.reshape(B, H, dv), o_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(st.reshape(B, H, dk, dv), S_ref, rtol=1e-12, atol=1e-12)
