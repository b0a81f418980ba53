"""CPU oracle for the fused PSD lift of queries and keys, in float64 (NumPy).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything under
``oracle/``. The library never does, and this code shares nothing with it.

The feature map is the rank-one PSD lift of the KATA page (section 2.2,
"Capacity theory"): a p-dimensional vector u becomes the p*p feature
psi(u) = vec(u u^T), whose inner products are squared inner products,
psi(u) . psi(w) = (u . w)^2, and whose norm is ||u||^2.

The fused entry point takes u (p = 16, so the feature dimension is 256) for the
queries and the keys and forms the features itself. Readings where the pages are
silent (each also listed in the design doc):
  * vec() is row-major: feature a*p + b is u_a u_b (u u^T is symmetric, so the
    column-major order gives the same vector);
  * u arrives in bf16, like every q/k input of the path, and each feature is the
    product of two bf16 values rounded to the nearest bf16 (ties to even), the
    dtype the unfused path's features have. The product of two bf16 values has at
    most 16 significant bits, so it is exact in float32 (and float64) within
    float32's normal range; the one rounding is the step to bf16.

With those features the recurrence is the plain KLA recurrence of kla_ref.
"""
from __future__ import annotations

import numpy as np

from . import kla_ref

__all__ = ["round_bf16_rne", "psd_features", "forward_psd"]


def round_bf16_rne(x) -> np.ndarray:
    """Nearest bf16 value (ties to even) of float32-representable values, as float64.

    A bf16 value is a float32 whose low 16 bits are zero. Rounding adds half of the
    dropped range (0x7FFF) plus the lowest kept bit, which breaks an exact tie toward an
    even kept mantissa, then clears the dropped bits.
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    bits = x32.view(np.uint32).astype(np.uint64)
    keep_lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + keep_lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    return rounded.view(np.float32).astype(np.float64)


def psd_features(u) -> np.ndarray:
    """psi(u) = vec(u u^T) on the last axis (KATA page, section 2.2), each entry rounded
    to bf16. u: [..., p] -> [..., p*p]."""
    u = np.asarray(u, dtype=np.float64)
    outer = u[..., :, None] * u[..., None, :]          # u_a u_b, exact for bf16 inputs
    flat = outer.reshape(*u.shape[:-1], u.shape[-1] * u.shape[-1])
    return round_bf16_rne(flat)


def forward_psd(uq, uk, v, log_alpha, eta, eps, init_state=None, beta_mode="kaczmarz"):
    """KLA forward with q = psi(u_q) and k = psi(u_k).

    uq, uk: [B, T, H, p]; v: [B, T, H, dv]; gates [B, T, H]; init_state [B, H, p*p, dv].
    Returns (o [B, T, H, dv], S_T [B, H, p*p, dv]).
    """
    return kla_ref.forward(psd_features(uq), psd_features(uk), v, log_alpha, eta, eps, init_state, beta_mode)
