"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bar: max|err| <= 1e-4 * RMS(ref) for fp32 inputs and <= 2e-2 * RMS(ref) for bf16
inputs, on the outputs and on the end state, element by element. Small cases
span several chunks and a ragged tail; full-size workloads are compared on
sampled heads that the C oracle computes over the whole sequence.
"""
import dataclasses
import os
import sys

import numpy as np
import pytest

import workloads as W
from oracle import cref, kla_ref
from tests.gpu_common import TOL, assert_close, err_over_rms, upload, upload_prefill

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import delta_rule_recurrence_kla_amd as kla  # noqa: E402


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_prefill(wl, path="auto", segments=0, init=None):
    q, k, v, la, eta, s0 = upload_prefill(wl)
    if init is not None:
        s0 = init
    out, fin = kla.chunk_fwd(q, k, v, la, eta, wl.eps, init_state=s0, chunk=wl.chunk, path=path, segments=segments)
    torch.cuda.synchronize()
    return out.cpu().numpy(), fin.cpu().numpy()


def oracle_prefill(wl):
    o, S = cref.forward(wl.q, wl.k, wl.v, wl.log_alpha, wl.eta, wl.eps, wl.init_state)
    B, T, H, dv = wl.B, wl.T, wl.H, wl.dv
    return o.reshape(B, H, T, dv).transpose(0, 2, 1, 3), S.reshape(B, H, wl.dk, dv)


# ---------------------------------------------------------------------------
# decode
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (256, 128), (128, 64), (64, 128), (256, 64)])
def test_decode_small(dtype, dk, dv):
    log(f"decode small dtype={dtype} dk={dk} dv={dv}")
    N, H, steps = 3, 5, 6
    S0 = W.make_decode_state(N, H, dk, dv, std=0.5, seed=3)
    S_dev = upload(S0, "f32")
    S_ref = S0.astype(np.float64)
    for s in range(steps):
        st = W.make_decode_step(s, N, H, dk, dv, dtype=dtype, seed=3)
        o = kla.decode_step(upload(st.q, dtype), upload(st.k, dtype), upload(st.v, dtype),
                            upload(st.log_alpha, "f32"), upload(st.eta, "f32"), S_dev, st.eps)
        o_ref, S_ref = kla_ref.decode_step(S_ref, st.q, st.k, st.v, st.log_alpha, st.eta, st.eps)
        assert_close(o.cpu().numpy(), o_ref, 1e-5, f"decode out step {s}")
    assert_close(S_dev.cpu().numpy(), S_ref, 1e-5, "decode state")


def test_decode_full_size_sampled():
    """Batched recurrent decode at its full shape: 256 sequences x 16 heads, dk=dv=128, all
    1024 successive steps of the workload; sampled heads checked against the C oracle at every
    step (outputs) and at the end (state). Step inputs are drawn a few steps ahead on worker
    threads (the draws are seeded per step, so the order of drawing does not matter)."""
    from concurrent.futures import ThreadPoolExecutor
    cfg = W.DECODE_CONFIG
    N, H, dk, dv = cfg["N"], cfg["H"], cfg["dk"], cfg["dv"]
    steps = cfg["steps"]
    log(f"case: decode full size N={N} H={H} steps={steps}")
    S0 = W.make_decode_state(N, H, dk, dv, std=cfg["state_std"], seed=0)
    S_dev = upload(S0, "f32")
    rng = np.random.default_rng(123)
    heads = [(int(a), int(b)) for a, b in zip(rng.integers(0, N, 48), rng.integers(0, H, 48))]
    heads = sorted(set(heads))
    S_ref = np.stack([S0[a, h] for a, h in heads]).astype(np.float64)
    worst = 0.0
    draw = lambda s: W.make_decode_step(s, N, H, dk, dv, dtype="bf16", seed=0)
    ahead = 8
    with ThreadPoolExecutor(ahead) as ex:
        pending = [ex.submit(draw, s) for s in range(min(ahead, steps))]
        for s in range(steps):
            st = pending.pop(0).result()
            if s + ahead < steps:
                pending.append(ex.submit(draw, s + ahead))
            o = kla.decode_step(upload(st.q, "bf16"), upload(st.k, "bf16"), upload(st.v, "bf16"),
                                upload(st.log_alpha, "f32"), upload(st.eta, "f32"), S_dev, st.eps)
            o_ref = cref.decode_step(S_ref, st.q, st.k, st.v, st.log_alpha, st.eta, st.eps, heads=heads)
            og = o.cpu().numpy()
            got = np.stack([og[a, h] for a, h in heads])
            worst = max(worst, err_over_rms(got, o_ref))
            assert worst <= TOL["bf16"], f"step {s}: {worst}"
            if s % 256 == 255:
                log(f"decode step {s + 1}: worst max|err|/RMS so far {worst:.2e}")
    Sg = S_dev.cpu().numpy()
    assert_close(np.stack([Sg[a, h] for a, h in heads]), S_ref, TOL["bf16"], "decode end state")
    log(f"decode full size ({steps} steps) worst max|err|/RMS = {worst:.2e}")


# ---------------------------------------------------------------------------
# prefill, small cases
def test_prefill_tiny_fp32_config():
    """Tiny CPU-checkable forward: B=1, H=2, T=256, dk=dv=64, fp32, seed 0, all outputs."""
    wl = W.make_prefill("tiny_f32", seed=0)
    log("prefill tiny fp32")
    o, S = run_prefill(wl)
    o_ref, S_ref = kla_ref.forward(wl.q, wl.k, wl.v, wl.log_alpha, wl.eta, wl.eps)
    e1 = assert_close(o, o_ref, TOL["f32"], "out")
    e2 = assert_close(S, S_ref, TOL["f32"], "final state")
    log(f"tiny fp32: out {e1:.2e} state {e2:.2e}")


SMALL = [(64, 64), (128, 128), (256, 128), (128, 64), (64, 128), (256, 64)]


@pytest.mark.parametrize("dk,dv", SMALL)
@pytest.mark.parametrize("T", [64, 200, 1000])
@pytest.mark.parametrize("path", ["sequential", "scan"])
def test_prefill_small_bf16(dk, dv, T, path):
    log(f"prefill bf16 dk={dk} dv={dv} T={T} path={path}")
    wl = W.make_prefill("lm_layer_4k", seed=T + dk, B=2, T=T, H=2, dk=dk, dv=dv, init_std=0.3)
    o, S = run_prefill(wl, path=path, segments=3)
    o_ref, S_ref = oracle_prefill(wl)
    assert_close(o, o_ref, TOL["bf16"] / 10, "out")
    assert_close(S, S_ref, TOL["bf16"] / 10, "final state")


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("T", [100, 640])
@pytest.mark.parametrize("path", ["sequential", "scan"])
def test_prefill_small_fp32(dk, dv, T, path):
    log(f"prefill fp32 dk={dk} dv={dv} T={T} path={path}")
    wl = W.make_prefill("tiny_f32", seed=T + dv, B=2, T=T, H=3, dk=dk, dv=dv, init_std=0.2)
    o, S = run_prefill(wl, path=path, segments=4)
    o_ref, S_ref = oracle_prefill(wl)
    assert_close(o, o_ref, TOL["f32"], "out")
    assert_close(S, S_ref, TOL["f32"], "final state")


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("bf16", 64, 64), ("bf16", 256, 64), ("f32", 128, 64)])
@pytest.mark.parametrize("path", ["sequential", "scan"])
def test_prefill_growth_gates(dtype, dk, dv, path):
    """Some log_alpha > 0 (accepted, not clamped): e^{g_r - g_i} exceeds 1 inside a chunk."""
    log(f"prefill growth gates {dtype} dk={dk} dv={dv} path={path}")
    name = "lm_layer_4k" if dtype == "bf16" else "tiny_f32"
    wl = W.make_prefill(name, seed=11 + dk, B=1, T=300, H=2, dk=dk, dv=dv, init_std=0.3)
    la = np.random.default_rng(7).uniform(-0.05, 0.04, wl.log_alpha.shape).astype(np.float32)
    wl = dataclasses.replace(wl, log_alpha=la)
    o, S = run_prefill(wl, path=path, segments=2)
    o_ref, S_ref = oracle_prefill(wl)
    assert_close(o, o_ref, TOL[dtype], "out")
    assert_close(S, S_ref, TOL[dtype], "final state")


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("bf16", 64, 64), ("bf16", 256, 128), ("f32", 64, 64)])
@pytest.mark.parametrize("B,H,T", [(1, 1, 1), (1, 3, 65), (3, 5, 130)])
def test_prefill_odd_grids(dtype, dk, dv, B, H, T):
    """One token, one token past a chunk, and batch x heads that fill no regular grid."""
    log(f"prefill odd grid {dtype} dk={dk} dv={dv} B={B} H={H} T={T}")
    name = "lm_layer_4k" if dtype == "bf16" else "tiny_f32"
    wl = W.make_prefill(name, seed=B * 100 + H * 10 + T % 7, B=B, T=T, H=H, dk=dk, dv=dv, init_std=0.3)
    for path in ("sequential", "scan"):
        o, S = run_prefill(wl, path=path, segments=2)
        o_ref, S_ref = oracle_prefill(wl)
        assert_close(o, o_ref, TOL[dtype], f"out ({path})")
        assert_close(S, S_ref, TOL[dtype], f"final state ({path})")


def _direct_mode_case(dtype, dk, dv, T, seed):
    """Keys of norm s in [0.6, 1.6] and eta in [0, 0.7): eta ||k||^2 < 1.8, so the direct write
    (beta = eta as given) stays non-expansive and the run is well conditioned."""
    name = "lm_layer_4k" if dtype == "bf16" else "tiny_f32"
    wl = W.make_prefill(name, seed=seed, B=2, T=T, H=2, dk=dk, dv=dv, init_std=0.3)
    rng = np.random.default_rng(seed)
    k = wl.k.astype(np.float64)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    k *= np.clip(np.exp(0.25 * rng.standard_normal(k.shape[:-1] + (1,))), 0.6, 1.6)
    k = k.astype(np.float32)
    if dtype == "bf16":
        k = W.round_to_bf16(k)
    eta = (0.7 * rng.uniform(0, 1, wl.eta.shape)).astype(np.float32)
    return dataclasses.replace(wl, k=k, eta=eta)


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("bf16", 64, 64), ("bf16", 256, 128),
                                         ("f32", 64, 64), ("f32", 128, 64)])
@pytest.mark.parametrize("path", ["sequential", "scan"])
def test_prefill_direct_beta_mode(dtype, dk, dv, path):
    """beta = eta as given (the Gated DeltaNet rule) through the same kernels, against the oracle's
    direct mode; and the two modes differ on these keys."""
    log(f"prefill direct beta {dtype} dk={dk} dv={dv} path={path}")
    wl = _direct_mode_case(dtype, dk, dv, 300, 31 + dk)
    q, k, v, la, eta, s0 = upload_prefill(wl)
    out, fin = kla.chunk_fwd(q, k, v, la, eta, wl.eps, init_state=s0, path=path, segments=3, beta_mode="direct")
    torch.cuda.synchronize()
    o_ref, S_ref = cref.forward(wl.q, wl.k, wl.v, wl.log_alpha, wl.eta, wl.eps, wl.init_state, beta_mode="direct")
    B, T, H = wl.B, wl.T, wl.H
    o_ref = o_ref.reshape(B, H, T, dv).transpose(0, 2, 1, 3)
    S_ref = S_ref.reshape(B, H, dk, dv)
    assert_close(out.cpu().numpy(), o_ref, TOL[dtype], "out")
    assert_close(fin.cpu().numpy(), S_ref, TOL[dtype], "final state")
    o_k, _ = oracle_prefill(wl)
    assert err_over_rms(o_k, o_ref) > 10 * TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_direct_beta_mode(dtype):
    log(f"decode direct beta {dtype}")
    rng = np.random.default_rng(41)
    N, H, dk, dv = 8, 4, 128, 128
    S0 = (0.3 * rng.standard_normal((N, H, dk, dv))).astype(np.float32)
    q = rng.standard_normal((N, H, dk)).astype(np.float32)
    k = rng.standard_normal((N, H, dk)).astype(np.float32)
    k *= (1.3 / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((N, H, dv)).astype(np.float32)
    la = np.log(rng.uniform(0.8, 1.0, (N, H))).astype(np.float32)
    eta = rng.uniform(0.1, 1.0, (N, H)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = (W.round_to_bf16(x) for x in (q, k, v))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    st = torch.from_numpy(S0).to(dev)
    out = kla.decode_step(*(torch.from_numpy(x).to(dev).to(tdt) for x in (q, k, v)),
                          torch.from_numpy(la).to(dev), torch.from_numpy(eta).to(dev), st, 1e-6,
                          beta_mode="direct")
    torch.cuda.synchronize()
    o_ref, S_ref = kla_ref.decode_step(S0, q, k, v, la, eta, 1e-6, beta_mode="direct")
    assert_close(out.cpu().numpy(), o_ref, TOL["f32"], "out")
    assert_close(st.cpu().numpy(), S_ref, TOL["f32"], "state")


def test_timing_hook_selects_one_kernel():
    """With a kernel selected, the hook records that kernel's launches and no other."""
    wl = W.make_prefill("lm_layer_4k", seed=3, B=1, T=256, H=2)
    q, k, v, la, eta, s0 = upload_prefill(wl)
    kla.timing_collect()
    kla.timing_select("kla_state_seq")
    kla.timing_enable(True)
    try:
        for _ in range(3):
            kla.chunk_fwd(q, k, v, la, eta, wl.eps, path="sequential")
        torch.cuda.synchronize()
    finally:
        kla.timing_enable(False)
        kla.timing_select(None)
    t = kla.timing_collect()
    assert set(t) == {"kla_state_seq"} and t["kla_state_seq"][0] == 3 and t["kla_state_seq"][1] > 0
    kla.timing_enable(True)
    kla.chunk_fwd(q, k, v, la, eta, wl.eps, path="sequential")
    torch.cuda.synchronize()
    kla.timing_enable(False)
    assert {"kla_prep", "kla_state_seq"} <= set(kla.timing_collect())


def test_prefill_psd_recipe_small():
    log("prefill psd small")
    wl = W.make_prefill("psd_lift_8k", seed=5, B=1, T=700, H=2)
    o, S = run_prefill(wl)
    o_ref, S_ref = oracle_prefill(wl)
    assert_close(o, o_ref, TOL["bf16"] / 10, "out")
    assert_close(S, S_ref, TOL["bf16"] / 10, "final state")


# ---------------------------------------------------------------------------
# invariants
def test_zero_length_copies_init():
    wl = W.make_prefill("lm_layer_4k", seed=1, B=2, T=0, H=3, init_std=1.0)
    q, k, v, la, eta, s0 = upload_prefill(wl)
    out, fin = kla.chunk_fwd(q, k, v, la, eta, wl.eps, init_state=s0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(fin.cpu().numpy(), wl.init_state)
    _, fin0 = kla.chunk_fwd(q, k, v, la, eta, wl.eps)
    torch.cuda.synchronize()
    assert np.all(fin0.cpu().numpy() == 0)


def test_split_prefill_equals_whole():
    """prefill(T) == prefill(T1) then prefill(T - T1) from its end state."""
    wl = W.make_prefill("lm_layer_4k", seed=2, B=2, T=640, H=2, init_std=0.1)
    q, k, v, la, eta, s0 = upload_prefill(wl)
    o, S = kla.chunk_fwd(q, k, v, la, eta, wl.eps, init_state=s0)
    T1 = 300
    sl = lambda x, a, b: x[:, a:b].contiguous()
    o1, S1 = kla.chunk_fwd(sl(q, 0, T1), sl(k, 0, T1), sl(v, 0, T1), sl(la, 0, T1), sl(eta, 0, T1), wl.eps, init_state=s0)
    o2, S2 = kla.chunk_fwd(sl(q, T1, 640), sl(k, T1, 640), sl(v, T1, 640), sl(la, T1, 640), sl(eta, T1, 640),
                           wl.eps, init_state=S1)
    torch.cuda.synchronize()
    on = o.cpu().numpy()
    assert_close(np.concatenate([o1.cpu().numpy(), o2.cpu().numpy()], 1), on, 2e-4, "split out")
    assert_close(S2.cpu().numpy(), S.cpu().numpy(), 2e-4, "split state")


def test_prefill_then_decode_equals_longer_prefill():
    """Decode continues from the prefill's end state: prefill(T) + 5 decode steps ==
    prefill(T + 5) on the last 5 outputs."""
    wl = W.make_prefill("lm_layer_4k", seed=4, B=2, T=133, H=2)
    q, k, v, la, eta, s0 = upload_prefill(wl)
    o, S = kla.chunk_fwd(q, k, v, la, eta, wl.eps)
    T1 = 128
    sl = lambda x: x[:, :T1].contiguous()
    _, St = kla.chunk_fwd(sl(q), sl(k), sl(v), sl(la), sl(eta), wl.eps)
    outs = []
    for t in range(T1, 133):
        outs.append(kla.decode_step(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
                                    la[:, t].contiguous(), eta[:, t].contiguous(), St, wl.eps))
    torch.cuda.synchronize()
    dec = np.stack([x.cpu().numpy() for x in outs], 1)
    assert_close(dec, o.cpu().numpy()[:, T1:], 2e-4, "decode after prefill")
    assert_close(St.cpu().numpy(), S.cpu().numpy(), 2e-4, "state after decode")


def test_sequential_equals_scan():
    wl = W.make_prefill("long_131k", seed=6, B=1, T=64 * 37 + 5, H=3, init_std=0.2)
    o1, S1 = run_prefill(wl, path="sequential")
    for segs in (2, 5, 37):
        o2, S2 = run_prefill(wl, path="scan", segments=segs)
        assert_close(o2, o1, 1e-3, f"scan({segs}) out")
        assert_close(S2, S1, 1e-3, f"scan({segs}) state")


@pytest.mark.parametrize("dk,dv", [(128, 128), (256, 128), (64, 64)])
def test_scan_zero_start_equals_explicit_zero_init(dk, dv):
    """Without an initial state the scan does not form segment 0's M (its map walk skips the
    identity columns and the fold skips the product). Passing an all-zero initial state takes
    the full route (M_0 formed, M_0 times zero added), so both must agree bit for bit; the
    no-init run must also match the oracle."""
    wl = W.make_prefill("long_131k", seed=8, B=2, T=64 * 23 + 17, H=2, dk=dk, dv=dv)
    log(f"case: zero-start scan dk={dk} dv={dv} T={wl.T}")
    zero = torch.zeros((wl.B, wl.H, dk, dv), dtype=torch.float32, device="cuda")
    for segs in (2, 4, 7):
        o1, S1 = run_prefill(wl, path="scan", segments=segs)
        o2, S2 = run_prefill(wl, path="scan", segments=segs, init=zero)
        assert np.array_equal(o1, o2) and np.array_equal(S1, S2), f"segments={segs}"
    o_ref, S_ref = oracle_prefill(wl)
    assert_close(o1, o_ref, TOL["bf16"], "out")
    assert_close(S1, S_ref, TOL["bf16"], "state")


def test_causality_and_determinism():
    wl = W.make_prefill("lm_layer_4k", seed=7, B=1, T=500, H=2)
    q, k, v, la, eta, _ = upload_prefill(wl)
    o_a, S_a = kla.chunk_fwd(q, k, v, la, eta, wl.eps)
    o_b, S_b = kla.chunk_fwd(q, k, v, la, eta, wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(S_a, S_b), "two runs differ"
    t = 300
    q2, k2, v2 = q.clone(), k.clone(), v.clone()
    q2[:, t + 1:] += 1
    k2[:, t + 1:] *= 2
    v2[:, t + 1:] -= 3
    o_c, _ = kla.chunk_fwd(q2, k2, v2, la, eta, wl.eps)
    torch.cuda.synchronize()
    assert torch.equal(o_c[:, : t + 1], o_a[:, : t + 1]), "outputs up to t changed"
    assert not torch.equal(o_c[:, t + 1:], o_a[:, t + 1:])


def test_final_state_may_alias_init():
    wl = W.make_prefill("lm_layer_4k", seed=8, B=2, T=300, H=2, init_std=0.3)
    q, k, v, la, eta, s0 = upload_prefill(wl)
    o_ref, S_ref = kla.chunk_fwd(q, k, v, la, eta, wl.eps, init_state=s0.clone())
    o, _ = kla.chunk_fwd(q, k, v, la, eta, wl.eps, init_state=s0, final_state=s0)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(s0, S_ref)


def test_exact_projection_self_check():
    """q = k with eta = 1: o_t = S_t^T k_t = v_t - (1 - beta_t ||k_t||^2) e_t, i.e. v_t up to eps
    (KLA page, "Theoretical derivation"); checked on PSD-lifted keys without the oracle."""
    wl = W.make_prefill("psd_lift_8k", seed=9, B=1, T=2048, H=4)
    q, k, v, la, eta, _ = upload_prefill(wl)
    o, _ = kla.chunk_fwd(k, k, v, la, eta, 0.0)
    torch.cuda.synchronize()
    e = err_over_rms(o.cpu().numpy(), wl.v)
    assert e < 2e-2, e


# ---------------------------------------------------------------------------
# full-size workloads, sampled heads
def _full_size(name, n_heads, path="auto"):
    wl = W.make_prefill(name, seed=0)
    log(f"full size {name}: B={wl.B} T={wl.T} H={wl.H} dk={wl.dk} dv={wl.dv} path={path}")
    q, k, v, la, eta, s0 = upload_prefill(wl)
    out, fin = kla.chunk_fwd(q, k, v, la, eta, wl.eps, init_state=s0, path=path)
    torch.cuda.synchronize()
    rng = np.random.default_rng(99)
    heads = sorted({(int(rng.integers(wl.B)), int(rng.integers(wl.H))) for _ in range(n_heads)})
    o_ref, S_ref = cref.forward(wl.q, wl.k, wl.v, wl.log_alpha, wl.eta, wl.eps, wl.init_state, heads=heads)
    got_o = np.stack([out[b, :, h].cpu().numpy() for b, h in heads])
    got_S = np.stack([fin[b, h].cpu().numpy() for b, h in heads])
    e1 = assert_close(got_o, o_ref, TOL[wl.dtype], f"{name} out")
    e2 = assert_close(got_S, S_ref, TOL[wl.dtype], f"{name} state")
    log(f"{name}: out {e1:.2e} state {e2:.2e} on {len(heads)} heads")
    return out


def test_full_lm_layer_4k():
    _full_size("lm_layer_4k", 12)


def test_full_psd_lift_8k():
    _full_size("psd_lift_8k", 6)


def test_full_long_131k():
    _full_size("long_131k", 3)
