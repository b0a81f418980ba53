"""The chunkwise backward, in float64, against the token-level gradient oracle (CPU).

A model for backward kernels to come, not part of the oracle or the library. Per chunk
(start state S0, chunk-local g = cumsum(log_alpha), Delta_ri = e^{g_r - g_i}, E = diag(e^g),
w = e^{g_C - g}, gamma = e^{g_C}) the forward of tests/test_chunk_algebra.py is
  A  = strict_lower(diag(beta) (Delta . K K^T)),   T' = (I + A)^-1 diag(beta),
  X  = V - E K S0,   U = T' X,   P = tril_incl(Delta . Q K^T),
  O  = E Q S0 + P U,   S1 = gamma S0 + K^T diag(w) U.
Reverse mode through these products, from dO and dS1, in the reverse order of the forward:
  S1:  dS0 += gamma dS1;  dgamma = <dS1, S0>;  dK += diag(w) U dS1^T;  dU += diag(w) K dS1;
       dw = rowsum(U . K dS1)
  O:   dS0 += Q^T E dO;  dQ += E dO S0^T;  deg += rowsum(dO . Q S0);  dP = tril_incl(dO U^T);
       dU += P^T dO
  P:   dQK = dP . Delta;  dQ += dQK K;  dK += dQK^T Q;  dDelta += dP . Q K^T
  U:   dT' = dU X^T;  dX = T'^T dU
  X:   dV = dX;  dK -= E dX S0^T;  dS0 -= K^T E dX;  deg -= rowsum(dX . K S0)
  T':  with Minv = (I + A)^-1:  dbeta += colsum(Minv . dT');  dA = strict_lower(-Minv^T (dT' diag(beta)) Minv^T)
  A:   dbeta += rowsum(dA . Delta . G);  dDelta += dA . beta_r G;  dG = dA . beta_r Delta;  dK += (dG + dG^T) K
  beta = eta / (n + eps):  deta = dbeta / (n + eps);  dK += 2 diag(-dbeta eta / (n + eps)^2) K
  decay:  dg += rowsum(dDelta . Delta) - colsum(dDelta . Delta) + deg . e^g - dw . w;
          dg_C += sum(dw . w) + dgamma gamma;  dlog_alpha = reverse cumsum of dg
Chunks are taken last to first, each with the end-state gradient its successor passes back.
"""
import numpy as np
import pytest

from oracle import kla_bwd
from tests.test_chunk_algebra import chunk_step


def chunk_backward(S0, Q, K, V, la, eta, eps, dO, dS1):
    C = len(la)
    g = np.cumsum(la)
    n = np.sum(K * K, 1)
    den = n + np.float64(np.float32(eps))
    beta = eta / den
    Dl = np.exp(g[:, None] - g[None, :])
    G = K @ K.T
    A = np.tril(beta[:, None] * Dl * G, -1)
    Minv = np.linalg.inv(np.eye(C) + A)
    Tp = Minv @ np.diag(beta)
    eg = np.exp(g)
    X = V - eg[:, None] * (K @ S0)
    U = Tp @ X
    QK = Q @ K.T
    incl = np.tril(np.ones((C, C)))
    P = incl * Dl * QK
    w = np.exp(g[-1] - g)
    gam = np.exp(g[-1])

    dS0 = gam * dS1
    dgam = np.sum(dS1 * S0)
    dK = (w[:, None] * U) @ dS1.T
    KdS1 = K @ dS1
    dU = w[:, None] * KdS1
    dw = np.sum(U * KdS1, 1)
    dS0 += Q.T @ (eg[:, None] * dO)
    dQ = eg[:, None] * (dO @ S0.T)
    deg = np.sum(dO * (Q @ S0), 1)
    dP = incl * (dO @ U.T)
    dU += P.T @ dO
    dQK = dP * Dl
    dQ += dQK @ K
    dK += dQK.T @ Q
    dDl = dP * QK
    dTp = dU @ X.T
    dX = Tp.T @ dU
    dV = dX
    dK -= eg[:, None] * (dX @ S0.T)
    dS0 -= K.T @ (eg[:, None] * dX)
    deg -= np.sum(dX * (K @ S0), 1)
    dbeta = np.sum(Minv * dTp, 0)
    dA = np.tril(-Minv.T @ (dTp * beta[None, :]) @ Minv.T, -1)
    dbeta += np.sum(dA * Dl * G, 1)
    dDl += dA * beta[:, None] * G
    dG = dA * beta[:, None] * Dl
    dK += (dG + dG.T) @ K
    deta = dbeta / den
    dK += 2.0 * (-dbeta * eta / den ** 2)[:, None] * K
    dg = np.sum(dDl * Dl, 1) - np.sum(dDl * Dl, 0) + deg * eg - dw * w
    dg[-1] += np.sum(dw * w) + dgam * gam
    dla = np.cumsum(dg[::-1])[::-1]
    return dict(dq=dQ, dk=dK, dv=dV, dlog_alpha=dla, deta=deta), dS0


def chunked_backward(q, k, v, la, eta, eps, S0, dO, dS_T, C):
    T = len(la)
    starts, S = [], S0.copy()
    for c0 in range(0, T, C):
        starts.append(S)
        sl = slice(c0, min(T, c0 + C))
        _, S = chunk_step(S, q[sl], k[sl], v[sl], la[sl], eta[sl], eps)
    out = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dlog_alpha", la), ("deta", eta))}
    dS = dS_T.copy()
    for ci, c0 in reversed(list(enumerate(range(0, T, C)))):
        sl = slice(c0, min(T, c0 + C))
        gr, dS = chunk_backward(starts[ci], q[sl], k[sl], v[sl], la[sl], eta[sl], eps, dO[sl], dS)
        for name in out:
            out[name][sl] = gr[name]
    out["dS0"] = dS
    return out


@pytest.mark.parametrize("C", [16, 64])
@pytest.mark.parametrize("T,dk,dv,seed", [(100, 8, 5, 0), (64 * 3, 16, 8, 1), (37, 6, 4, 2)])
def test_chunked_backward_equals_token_gradients(T, dk, dv, C, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk)) * np.exp(0.5 * rng.standard_normal((T, 1)))
    v = rng.standard_normal((T, dv))
    la = np.log(rng.uniform(0.6, 1.0, T))
    eta = rng.uniform(0.1, 1.0, T)
    S0 = 0.3 * rng.standard_normal((dk, dv))
    dO = rng.standard_normal((T, dv))
    dS_T = rng.standard_normal((dk, dv))
    eps = 1e-6
    ref = kla_bwd.backward(q, k, v, la, eta, eps, dO, dS_T, S0)
    got = chunked_backward(q, k, v, la, eta, eps, S0, dO, dS_T, C)
    for name in ("dq", "dk", "dv", "dlog_alpha", "deta", "dS0"):
        scale = max(np.max(np.abs(ref[name])), 1e-30)
        assert np.max(np.abs(got[name] - ref[name])) <= 1e-9 * scale, name
