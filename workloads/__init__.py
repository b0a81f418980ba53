"""Seeded synthetic inputs for the KLA forward path.

This module only draws random numbers and shapes them into the five workloads
(value distributions, bf16 rounding, layouts). It holds none of the method's
arithmetic, so both the CPU oracle (``oracle/``) and the HIP path
(``delta_rule_recurrence_kla_amd``) can be fed from it without sharing code.

Layouts (the order of the library's size arguments):
  q, k      [B, T, H, dk]   float32 arrays holding bf16-exact values for bf16 workloads
  v         [B, T, H, dv]
  log_alpha [B, T, H]       float32, per-token decay gate in log space
  eta       [B, T, H]       float32, per-token relaxation gate
  state     [B, H, dk, dv]  float32, dv fastest

Every workload is synthetic; no dataset is read. The draw order within each
recipe is fixed, so a seed determines every value.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

__all__ = [
    "PrefillInputs",
    "DecodeInputs",
    "round_to_bf16",
    "bf16_bits",
    "make_prefill",
    "make_decode_state",
    "make_decode_step",
    "make_decode_steps",
    "psd_lift",
    "PREFILL_CONFIGS",
    "DECODE_CONFIG",
]


# ---------------------------------------------------------------------------
# bf16 rounding (round to nearest, ties to even), done on the float32 bit pattern
# ---------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns of float32 ``x`` rounded to nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array holding ``x`` rounded to the nearest bf16 value (ties to even)."""
    b = bf16_bits(x).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def _logsigmoid(x: np.ndarray) -> np.ndarray:
    # log(1/(1+e^-x)) = -log1p(e^-x), written to avoid overflow for large |x|
    return np.where(x >= 0, -np.log1p(np.exp(-x)), x - np.log1p(np.exp(x))).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-30))).astype(np.float32)


def psd_lift(u: np.ndarray) -> np.ndarray:
    """Rank-one PSD feature of the KATA page (section 2.2, capacity theory):
    psi(u) = vec(u u^T), flattened row-major, so a p-vector becomes p*p features."""
    u = np.asarray(u, dtype=np.float32)
    p = u.shape[-1]
    return (u[..., :, None] * u[..., None, :]).reshape(*u.shape[:-1], p * p).astype(np.float32)


# ---------------------------------------------------------------------------
# Prefill workloads
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class PrefillInputs:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    chunk: int
    dtype: str  # "f32" or "bf16": the dtype q, k, v are handed to the kernels in
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    log_alpha: np.ndarray
    eta: np.ndarray
    eps: float
    init_state: Optional[np.ndarray]

    def head_slice(self, heads) -> "PrefillInputs":
        """The same workload restricted to the listed (b, h) pairs, each as its own batch row."""
        heads = list(heads)
        def take(a):
            return np.stack([a[b, :, h] for (b, h) in heads])[:, :, None]
        init = None
        if self.init_state is not None:
            init = np.stack([self.init_state[b, h] for (b, h) in heads])[:, None]
        return PrefillInputs(self.name + "[heads]", len(heads), self.T, 1, self.dk, self.dv,
                             self.chunk, self.dtype, take(self.q), take(self.k), take(self.v),
                             take(self.log_alpha), take(self.eta), self.eps, init)


# Shapes of the five workloads. Config names describe what each one is.
PREFILL_CONFIGS = {
    # tiny CPU-checkable forward, fp32
    "tiny_f32": dict(B=1, T=256, H=2, dk=64, dv=64, chunk=64, dtype="f32", recipe="gaussian"),
    # one 0.4B-LM-shaped layer, chunked prefill
    "lm_layer_4k": dict(B=8, T=4096, H=16, dk=128, dv=128, chunk=64, dtype="bf16", recipe="l2norm"),
    # long-context prefill, few heads (exercises the associative-scan path)
    "long_131k": dict(B=1, T=131072, H=16, dk=128, dv=128, chunk=64, dtype="bf16", recipe="gaussian"),
    # PSD-lifted keys, p=16 -> dk=256, exact Kaczmarz projection without decay
    "psd_lift_8k": dict(B=4, T=8192, H=8, dk=256, dv=128, chunk=64, dtype="bf16", recipe="psd"),
}


def make_prefill(name: str = "tiny_f32", seed: int = 0, *, recipe: Optional[str] = None,
                 init_std: float = 0.0, **overrides) -> PrefillInputs:
    """Draw one prefill workload.

    recipes (value distributions, all N(mean, std)):
      gaussian: q, k ~ N(0,1); each k row times exp(0.5*N(0,1)) (lognormal(0, 0.5));
                v ~ N(0,1); log_alpha = logsigmoid(N(3,1)); eta = sigmoid(N(0,1))
      l2norm:   q, k ~ N(0,1), each row L2-normalised, then times its own lognormal(0, 0.5);
                v, gates as gaussian
      psd:      u_q, u_k ~ N(0, I_p) unit-normalised, q = psi(u_q), k = psi(u_k) with
                p = sqrt(dk); v ~ N(0,1); log_alpha = 0; eta = 1
    eps = 1e-6 throughout. ``init_std`` > 0 draws a N(0, init_std) initial state last.
    Any shape field may be overridden (e.g. T=100 for a ragged small case).
    """
    cfg = dict(PREFILL_CONFIGS[name])
    cfg.update(overrides)
    if recipe is not None:
        cfg["recipe"] = recipe
    B, T, H, dk, dv = cfg["B"], cfg["T"], cfg["H"], cfg["dk"], cfg["dv"]
    rng = np.random.default_rng(seed)
    f32 = np.float32
    r = cfg["recipe"]
    if r in ("gaussian", "l2norm"):
        q = rng.standard_normal((B, T, H, dk), dtype=f32)
        k = rng.standard_normal((B, T, H, dk), dtype=f32)
        if r == "l2norm":
            q = _l2_normalise(q) * np.exp(f32(0.5) * rng.standard_normal((B, T, H, 1), dtype=f32))
            k = _l2_normalise(k) * np.exp(f32(0.5) * rng.standard_normal((B, T, H, 1), dtype=f32))
        else:
            k = k * np.exp(f32(0.5) * rng.standard_normal((B, T, H, 1), dtype=f32))
        v = rng.standard_normal((B, T, H, dv), dtype=f32)
        log_alpha = _logsigmoid(f32(3.0) + rng.standard_normal((B, T, H), dtype=f32))
        eta = _sigmoid(rng.standard_normal((B, T, H), dtype=f32))
    elif r == "psd":
        p = int(round(np.sqrt(dk)))
        assert p * p == dk, "psd recipe needs a square dk"
        uq = _l2_normalise(rng.standard_normal((B, T, H, p), dtype=f32))
        uk = _l2_normalise(rng.standard_normal((B, T, H, p), dtype=f32))
        q = psd_lift(uq)
        k = psd_lift(uk)
        v = rng.standard_normal((B, T, H, dv), dtype=f32)
        log_alpha = np.zeros((B, T, H), f32)
        eta = np.ones((B, T, H), f32)
    else:
        raise ValueError(f"unknown recipe {r!r}")
    init = None
    if init_std > 0:
        init = (f32(init_std) * rng.standard_normal((B, H, dk, dv), dtype=f32)).astype(f32)
    if cfg["dtype"] == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return PrefillInputs(name, B, T, H, dk, dv, cfg["chunk"], cfg["dtype"],
                         np.ascontiguousarray(q, f32), np.ascontiguousarray(k, f32),
                         np.ascontiguousarray(v, f32), np.ascontiguousarray(log_alpha, f32),
                         np.ascontiguousarray(eta, f32), 1e-6, init)


# ---------------------------------------------------------------------------
# PSD workload in unlifted form: the p-wide u vectors themselves (for the fused lift)
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class PsdInputs:
    B: int
    T: int
    H: int
    p: int
    dv: int
    uq: np.ndarray         # [B, T, H, p], bf16-exact values
    uk: np.ndarray         # [B, T, H, p], bf16-exact values
    v: np.ndarray          # [B, T, H, dv], bf16-exact values
    log_alpha: np.ndarray  # [B, T, H]
    eta: np.ndarray        # [B, T, H]
    eps: float
    init_state: Optional[np.ndarray]  # [B, H, p*p, dv] or None


def make_psd_u(seed: int = 0, *, B: int = 4, T: int = 8192, H: int = 8, p: int = 16, dv: int = 128,
               gates: str = "psd", init_std: float = 0.0) -> PsdInputs:
    """The PSD workload's inputs before the lift: u_q, u_k ~ N(0, I_p) unit-normalised, then
    rounded to bf16; v ~ N(0,1) in bf16. gates "psd": log_alpha = 0, eta = 1 (the workload's
    exact projection without decay); "gaussian": log_alpha = logsigmoid(N(3,1)),
    eta = sigmoid(N(0,1)). eps = 1e-6. Defaults are the full PSD workload's shape."""
    rng = np.random.default_rng(seed)
    f32 = np.float32
    uq = round_to_bf16(_l2_normalise(rng.standard_normal((B, T, H, p), dtype=f32)))
    uk = round_to_bf16(_l2_normalise(rng.standard_normal((B, T, H, p), dtype=f32)))
    v = round_to_bf16(rng.standard_normal((B, T, H, dv), dtype=f32))
    if gates == "psd":
        log_alpha = np.zeros((B, T, H), f32)
        eta = np.ones((B, T, H), f32)
    elif gates == "gaussian":
        log_alpha = _logsigmoid(f32(3.0) + rng.standard_normal((B, T, H), dtype=f32))
        eta = _sigmoid(rng.standard_normal((B, T, H), dtype=f32))
    else:
        raise ValueError(f"unknown gates {gates!r}")
    init = None
    if init_std > 0:
        init = (f32(init_std) * rng.standard_normal((B, H, p * p, dv), dtype=f32)).astype(f32)
    c = lambda a: np.ascontiguousarray(a, f32)
    return PsdInputs(B, T, H, p, dv, c(uq), c(uk), c(v), c(log_alpha), c(eta), 1e-6, init)


# ---------------------------------------------------------------------------
# Decode workload: N sequences x H heads, fresh single-token inputs every step
# ---------------------------------------------------------------------------
DECODE_CONFIG = dict(N=256, H=16, dk=128, dv=128, steps=1024, state_std=0.02, dtype="bf16")


@dataclasses.dataclass
class DecodeInputs:
    q: np.ndarray          # [N, H, dk]
    k: np.ndarray          # [N, H, dk]
    v: np.ndarray          # [N, H, dv]
    log_alpha: np.ndarray  # [N, H]
    eta: np.ndarray        # [N, H]
    eps: float


def make_decode_state(N: int = 256, H: int = 16, dk: int = 128, dv: int = 128,
                      std: float = 0.02, seed: int = 0) -> np.ndarray:
    """Initial decode state, N(0, std) per entry, float32 [N, H, dk, dv]."""
    rng = np.random.default_rng(seed)
    return (np.float32(std) * rng.standard_normal((N, H, dk, dv), dtype=np.float32)).astype(np.float32)


def make_decode_step(step: int, N: int = 256, H: int = 16, dk: int = 128, dv: int = 128,
                     dtype: str = "bf16", seed: int = 0) -> DecodeInputs:
    """Inputs of decode step ``step``: q, v ~ N(0,1); k ~ N(0,1) L2-normalised (in fp32,
    before bf16 rounding); log_alpha = logsigmoid(N(3,1)); eta = sigmoid(N(0,1))."""
    rng = np.random.default_rng([seed, step])
    f32 = np.float32
    q = rng.standard_normal((N, H, dk), dtype=f32)
    k = _l2_normalise(rng.standard_normal((N, H, dk), dtype=f32))
    v = rng.standard_normal((N, H, dv), dtype=f32)
    la = _logsigmoid(f32(3.0) + rng.standard_normal((N, H), dtype=f32))
    eta = _sigmoid(rng.standard_normal((N, H), dtype=f32))
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return DecodeInputs(q, k, v, la, eta, 1e-6)


def make_decode_steps(steps: int, **kw) -> DecodeInputs:
    """Inputs of steps 0..steps-1 stacked on a leading axis."""
    per = [make_decode_step(s, **kw) for s in range(steps)]
    return DecodeInputs(*(np.stack([getattr(p, f) for p in per]) for f in ("q", "k", "v", "log_alpha", "eta")),
                        per[0].eps)


# ---------------------------------------------------------------------------
# Log-linear decode: per-level output weights and bucket states
# ---------------------------------------------------------------------------
# 256 sequences x 16 heads at 32K context (the KLA page measures decode at a 32K-token
# context): 16 levels cover positions below 2^15; the timed steps are the last 1024
# positions before 32768.
LOGLINEAR_DECODE_CONFIG = dict(N=256, H=16, dk=128, dv=128, levels=16, t0=32768 - 1024, steps=1024,
                               state_std=0.02, dtype="bf16")


def make_loglinear_lambda(step: int, N: int = 256, H: int = 16, levels: int = 16, seed: int = 0) -> np.ndarray:
    """Weights lambda^(l) of decode step ``step``: sigmoid(N(0,1)) per sequence, head and level,
    float32 [N, H, levels]; drawn from their own stream, so the step's q, k, v and gates are the
    same as make_decode_step's."""
    rng = np.random.default_rng([seed, step, 1])
    return _sigmoid(rng.standard_normal((N, H, levels), dtype=np.float32))


def make_loglinear_states(N: int = 256, H: int = 16, levels: int = 16, dk: int = 128, dv: int = 128,
                          std: float = 0.02, seed: int = 0) -> np.ndarray:
    """Bucket states to start a log-linear decode from, N(0, std) in every slot, float32
    [N, H, levels, dk, dv] (slots of levels that are empty at the start position are never read)."""
    rng = np.random.default_rng([seed, 2])
    return (np.float32(std) * rng.standard_normal((N, H, levels, dk, dv), dtype=np.float32)).astype(np.float32)


def make_bwd_grads(B: int, T: int, H: int, dk: int, dv: int, seed: int = 0, std: float = 1.0):
    """Upstream gradients for the prefill backward: d loss / d out ~ N(0, std) float32
    [B, T, H, dv] and d loss / d final state ~ N(0, std) float32 [B, H, dk, dv], from their own
    stream (the forward inputs of the same seed are unchanged)."""
    rng = np.random.default_rng([seed, 3])
    f = np.float32
    d_out = (f(std) * rng.standard_normal((B, T, H, dv), dtype=f)).astype(f)
    d_fin = (f(std) * rng.standard_normal((B, H, dk, dv), dtype=f)).astype(f)
    return d_out, d_fin
