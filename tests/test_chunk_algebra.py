"""The chunk algebra the kernels implement, in float64, against the token-by-token oracle.

Inside a chunk with start state S0, g_r = sum_{j<=r} log_alpha_j and u_i = beta_i e_i,
unrolling the KLA update rule gives (I + A) U = diag(beta) (V - diag(e^g) K S0), with
A_ri = beta_r e^{g_r-g_i} (k_r . k_i) for i < r. Hence, with T' = (I + A)^-1 diag(beta):
  U   = T' (V - diag(e^g) K S0)
  O   = diag(e^g) Q S0 + P U,   P_ri = e^{g_r-g_i} (q_r . k_i) for i <= r
  S_C = e^{g_C} S0 + K^T diag(e^{g_C-g}) U.
A run of chunks is an affine map S_end = M S_start + N; composing the maps of
consecutive segments reproduces the serial walk (the associative scan of the KATA
page, section 2.3, and the HLA page, section 4).

This file is a model for the kernels, not part of either the oracle or the library.
"""
import numpy as np
import pytest

import workloads as W
from oracle import kla_ref


def chunk_step(S0, Q, K, V, la, eta, eps):
    C = len(la)
    g = np.cumsum(la)
    beta = eta / (np.sum(K * K, 1) + np.float32(eps))
    D = np.exp(g[:, None] - g[None, :])
    A = np.tril(beta[:, None] * D * (K @ K.T), -1)
    Tp = np.linalg.solve(np.eye(C) + A, np.diag(beta))
    U = Tp @ (V - np.exp(g)[:, None] * (K @ S0))
    P = np.tril(D * (Q @ K.T))
    O = np.exp(g)[:, None] * (Q @ S0) + P @ U
    S = np.exp(g[-1]) * S0 + K.T @ (np.exp(g[-1] - g)[:, None] * U)
    return O, S


def chunked_forward(q, k, v, la, eta, eps, S0, C):
    T = len(la)
    S = S0.copy()
    outs = []
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        O, S = chunk_step(S, q[sl], k[sl], v[sl], la[sl], eta[sl], eps)
        outs.append(O)
    return np.concatenate(outs), S


def segment_map(q, k, v, la, eta, eps, C, dk):
    """[M | N] of a run of chunks: walk the augmented state [I | 0] with zero values in the identity part."""
    dv = v.shape[1]
    S = np.concatenate([np.eye(dk), np.zeros((dk, dv))], 1)
    Vaug = np.concatenate([np.zeros((len(la), dk)), v], 1)
    for c0 in range(0, len(la), C):
        sl = slice(c0, min(len(la), c0 + C))
        _, S = chunk_step(S, q[sl], k[sl], Vaug[sl], la[sl], eta[sl], eps)
    return S[:, :dk], S[:, dk:]


def _head(name, seed, T, dk, dv):
    wl = W.make_prefill(name, seed=seed, B=1, T=T, H=1, dk=dk, dv=dv, init_std=0.3)
    f = lambda a: a[0, :, 0].astype(np.float64)
    return f(wl.q), f(wl.k), f(wl.v), f(wl.log_alpha), f(wl.eta), wl.eps, wl.init_state[0, 0].astype(np.float64), wl


@pytest.mark.parametrize("C", [16, 64])
@pytest.mark.parametrize("name,T,dk,dv", [("tiny_f32", 200, 32, 16), ("lm_layer_4k", 300, 64, 32),
                                          ("psd_lift_8k", 130, 16, 8)])
def test_chunk_form_equals_recurrence(name, T, dk, dv, C):
    q, k, v, la, eta, eps, S0, wl = _head(name, 1, T, dk, dv)
    o_ref, S_ref = kla_ref.forward(wl.q, wl.k, wl.v, wl.log_alpha, wl.eta, eps, wl.init_state)
    o, S = chunked_forward(q, k, v, la, eta, eps, S0, C)
    scale = np.sqrt(np.mean(o_ref ** 2))
    assert np.max(np.abs(o - o_ref[0, :, 0])) < 1e-10 * max(scale, 1)
    assert np.max(np.abs(S - S_ref[0, 0])) < 1e-10


def test_growth_gates_need_the_unclamped_decay():
    """log_alpha > 0 is accepted (not clamped), so e^{g_r - g_i} can exceed 1 inside a chunk;
    the chunk form with the exact factor matches the recurrence, one capped at 1 does not."""
    q, k, v, la, eta, eps, S0, wl = _head("lm_layer_4k", 5, 200, 32, 16)
    la = np.random.default_rng(3).uniform(-0.05, 0.04, la.shape)
    o_ref, S_ref = kla_ref.forward(wl.q, wl.k, wl.v, la[None, :, None].astype(np.float32), wl.eta, eps,
                                   wl.init_state)
    la = la.astype(np.float32).astype(np.float64)
    o, S = chunked_forward(q, k, v, la, eta, eps, S0, 64)
    scale = np.sqrt(np.mean(o_ref ** 2))
    assert np.max(np.abs(o - o_ref[0, :, 0])) < 1e-10 * max(scale, 1)
    assert np.max(np.abs(S - S_ref[0, 0])) < 1e-10

    def clamped_step(S0, Q, K, V, la, eta, eps):
        g = np.cumsum(la)
        beta = eta / (np.sum(K * K, 1) + np.float32(eps))
        D = np.exp(np.minimum(g[:, None] - g[None, :], 0))
        A = np.tril(beta[:, None] * D * (K @ K.T), -1)
        U = np.linalg.solve(np.eye(len(la)) + A, np.diag(beta)) @ (V - np.exp(g)[:, None] * (K @ S0))
        return np.exp(g)[:, None] * (Q @ S0) + np.tril(D * (Q @ K.T)) @ U

    o_c = clamped_step(S0, q[:64], k[:64], v[:64], la[:64], eta[:64], eps)
    assert np.max(np.abs(o_c - o_ref[0, :64, 0])) > 1e-3 * scale


def test_padding_with_identity_steps_changes_nothing():
    """A ragged chunk padded with k = q = v = 0, log_alpha = 0, eta = 0 gives the same result."""
    q, k, v, la, eta, eps, S0, _ = _head("lm_layer_4k", 2, 100, 32, 16)
    o1, S1 = chunked_forward(q, k, v, la, eta, eps, S0, 64)
    pad = 28
    z = lambda a: np.concatenate([a, np.zeros((pad,) + a.shape[1:])])
    o2, S2 = chunked_forward(z(q), z(k), z(v), z(la), z(eta), eps, S0, 64)
    np.testing.assert_allclose(o2[:100], o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("segments", [2, 3, 5])
def test_segment_maps_compose_to_serial(segments):
    q, k, v, la, eta, eps, S0, _ = _head("lm_layer_4k", 3, 64 * 10, 32, 16)
    dk = 32
    o_ser, S_ser = chunked_forward(q, k, v, la, eta, eps, S0, 64)
    L = -(-10 // segments) * 64
    bounds = [(s, min(640, s + L)) for s in range(0, 640, L)]
    # phase 1: maps of all but the last segment; phase 2: fold; phase 3: walk each segment from its start
    starts = [S0]
    for (a, b) in bounds[:-1]:
        M, N = segment_map(q[a:b], k[a:b], v[a:b], la[a:b], eta[a:b], eps, 64, dk)
        starts.append(M @ starts[-1] + N)
    outs = []
    for (a, b), St in zip(bounds, starts):
        o, S_end = chunked_forward(q[a:b], k[a:b], v[a:b], la[a:b], eta[a:b], eps, St, 64)
        outs.append(o)
    np.testing.assert_allclose(np.concatenate(outs), o_ser, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(S_end, S_ser, rtol=1e-10, atol=1e-10)


def test_residual_form_equals_wy_form():
    """U = T'(V - diag(e^g) K S0) equals the W/U~ form U~ - W S0 with W = T' diag(e^g) K, U~ = T' V."""
    q, k, v, la, eta, eps, S0, _ = _head("lm_layer_4k", 4, 64, 32, 16)
    g = np.cumsum(la)
    beta = eta / (np.sum(k * k, 1) + np.float32(eps))
    A = np.tril(beta[:, None] * np.exp(g[:, None] - g[None, :]) * (k @ k.T), -1)
    Tp = np.linalg.solve(np.eye(64) + A, np.diag(beta))
    U1 = Tp @ (v - np.exp(g)[:, None] * (k @ S0))
    Wm = Tp @ (np.exp(g)[:, None] * k)
    U2 = Tp @ v - Wm @ S0
    np.testing.assert_allclose(U1, U2, rtol=1e-12, atol=1e-12)
