"""GPU parity of the scan's backward pass (fwmem_scan_bwd) against the oracle's
scan_backward: every gradient (q, k, v, beta, lambda, the initial state and the carried
key) for the delta, inner and additive rules, phi identity and elu+1, bf16 and float32
inputs, carried and fresh states, ragged chunk tails, a lone no-op step and T = 0.

With float32 inputs every product runs in float32 and every gradient is held to the
float32 bar (1e-4). With bf16 inputs the chunk-parallel kernels (delta, inner and additive
rules with a scalar decay, no normaliser) carry every operand that is not an exact bf16
input as a bf16 hi + lo pair, about 16 bits of each factor, as the split forward kernels
do: those gradients are held to 1e-3 of rms, inside the 2e-2 bound for bf16 inputs. The
token-serial kernel (per-channel lambda, the per-value-channel rule, the normaliser) stays
float32 and keeps the float32 bar."""
import numpy as np
import pytest

from linear_attention_scan_amd import fwmem as F
from linear_attention_scan_amd import workloads as wl
from oracle import fwmem_oracle as orc
from tests.gpu_helpers import TOL, dev_tensor, f32_tensor, make_state, say

pytestmark = pytest.mark.gpu

RULES = {"delta": wl.RULE_DELTA, "inner": wl.RULE_INNER, "additive": wl.RULE_ADDITIVE}
TOL_SPLIT = 1e-3


def _tol(w):
    """The bar for w's gradients: 1e-3 where the split-operand chunked kernels serve it."""
    split = (w.dtype == "bf16" and w.rule in (wl.RULE_DELTA, wl.RULE_INNER, wl.RULE_ADDITIVE)
             and not w.per_channel and not getattr(w, "znorm", False))
    return TOL_SPLIT if split else TOL["f32"]


def _problem(rule, phi, dtype, dk, dv, T, carried, seed, B=2, H=2, lam_kind=None, beta_kind=None,
             per_channel=False):
    r = RULES[rule]
    if lam_kind is None:
        lam_kind = "gamma" if r == wl.RULE_ADDITIVE else "softplus"
    if beta_kind is None:
        beta_kind = "sigmoid" if r == wl.RULE_ADDITIVE else "two_sigmoid"
    w = wl.make_scan(B=B, H=H, T=T, dk=dk, dv=dv, dtype=dtype, rule=r,
                     phi=wl.PHI_ELU1 if phi == "elu1" else wl.PHI_IDENTITY,
                     beta_kind=beta_kind, lam_kind=lam_kind, lam_mu=-3.0, per_channel=per_channel,
                     normalise_qk=phi != "elu1", s0_std=0.1 if carried else None, seed=seed)
    rng = np.random.default_rng(seed + 1000)
    dO = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    dS = (rng.standard_normal((B, H, dk, dv)) * 0.3).astype(np.float32)
    xprev0 = has0 = None
    if carried and r != wl.RULE_ADDITIVE:
        kp = rng.standard_normal((B, H, dk)).astype(np.float32)
        kp /= np.linalg.norm(kp, axis=-1, keepdims=True)
        xprev0 = np.where(kp > 0, kp + 1.0, np.exp(kp)).astype(np.float32) if phi == "elu1" else kp
        has0 = np.ones((B, H), dtype=np.int32)
    return w, dO, dS, xprev0, has0


def _run(w, dO, dS, xprev0, has0, phi, carried, with_dS=True):
    flags = (F.PHI_ELU1 if phi == "elu1" else 0) | (F.LAMBDA_PER_CHANNEL if w.per_channel else 0)
    S_in = None
    if carried:
        S_in = make_state(w.B, w.H, w.dk, w.dv, S=w.S0, xprev=xprev0, has=has0)
    gS = make_state(w.B, w.H, w.dk, w.dv, S=dS) if with_dS else None
    g = F.scan_bwd(dev_tensor(w.q, w.dtype), dev_tensor(w.k, w.dtype), dev_tensor(w.v, w.dtype),
                   f32_tensor(w.beta), f32_tensor(w.lam), f32_tensor(dO), rule=w.rule,
                   flags=flags, eps=w.eps, S_in=S_in, grad_S_out=gS)
    ref = orc.scan_backward(w.q, w.k, w.v, w.beta, w.lam, dO, dS if with_dS else None,
                            rule=w.rule, phi_kind=phi, eps=w.eps, per_channel=w.per_channel,
                            S0=w.S0 if carried else None,
                            xprev0=xprev0, has0=has0)
    return g, ref, w


def _compare(g, ref, w, tol=None):
    tol = _tol(w) if tol is None else tol
    got = {"q": g["q"], "k": g["k"], "v": g["v"], "beta": g["beta"], "lam": g["lam"],
           "S0": g["state"].S, "xprev0": g["state"].x_prev}
    errs = {}
    for name, x in got.items():
        if ref[name] is None:
            assert x is None, name
            continue
        errs[name] = orc.relerr(x.cpu().numpy().astype(np.float64), ref[name])
    say("    " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for name, e in errs.items():
        assert e <= tol, f"grad {name}: {e:.3e} > {tol}"
    assert np.all(g["state"].has_prev.cpu().numpy() == 0)


@pytest.mark.parametrize("rule,phi,dtype,dk,dv,T,carried", [
    ("delta", "identity", "bf16", 128, 128, 150, True),
    ("delta", "identity", "bf16", 128, 128, 150, False),
    ("delta", "elu1", "f32", 64, 128, 100, False),
    ("delta", "identity", "f32", 128, 64, 64, True),
    ("delta", "elu1", "bf16", 64, 64, 200, True),
    ("inner", "identity", "bf16", 64, 64, 130, True),
    ("inner", "elu1", "bf16", 128, 128, 90, False),
    ("inner", "identity", "f32", 64, 128, 65, True),
    ("additive", "identity", "bf16", 128, 128, 150, True),
    ("additive", "elu1", "f32", 64, 64, 77, False),
    ("additive", "elu1", "bf16", 128, 64, 129, True),
])
def test_backward_matches_oracle(rule, phi, dtype, dk, dv, T, carried):
    seed = (dk + dv + T) * 7 + carried
    say(f"[bwd] {rule} {phi} {dtype} dk={dk} dv={dv} T={T} carried={carried}")
    w, dO, dS, x0, h0 = _problem(rule, phi, dtype, dk, dv, T, carried, seed)
    _compare(*_run(w, dO, dS, x0, h0, phi, carried))


@pytest.mark.parametrize("rule,phi,dtype,dk,dv,T,carried", [
    ("delta", "identity", "bf16", 128, 128, 100, True),
    ("delta", "elu1", "f32", 64, 128, 70, False),
    ("inner", "identity", "bf16", 128, 64, 97, True),
    ("inner", "elu1", "f32", 64, 64, 33, False),
    ("additive", "elu1", "bf16", 128, 128, 96, True),
    ("additive", "identity", "f32", 64, 128, 31, False),
])
def test_backward_per_channel_lambda(rule, phi, dtype, dk, dv, T, carried):
    """lambda [B,H,T,dk]: per-row decays; for the ridge rules the denominator's largest
    lambda_i takes its gradient. Chunks are 32 tokens here, so T spans several with a
    ragged tail."""
    seed = (dk + dv + T) * 5 + carried
    say(f"[bwd pc] {rule} {phi} {dtype} dk={dk} dv={dv} T={T} carried={carried}")
    w, dO, dS, x0, h0 = _problem(rule, phi, dtype, dk, dv, T, carried, seed, per_channel=True)
    _compare(*_run(w, dO, dS, x0, h0, phi, carried))


def test_backward_per_channel_tied_maximum():
    """Several channels share the largest lambda: the denominator's gradient goes to the
    first of them, as in the oracle."""
    say("[bwd pc] tied maximum")
    w, dO, dS, x0, h0 = _problem("delta", "identity", "f32", 64, 64, 40, True, 21, per_channel=True)
    w.lam[..., 5] = w.lam[..., 17] = w.lam[..., 60] = 5.0   # above every softplus(N(-3, 1)) draw
    _compare(*_run(w, dO, dS, x0, h0, "identity", True))


@pytest.mark.parametrize("rule", ["delta", "inner", "additive"])
def test_backward_default_gates(rule):
    """lambda absent (ridge 0 / retention 1) and, for the additive rule, beta absent (write
    scale 1): their gradients are not asked for and the rest still match."""
    say(f"[bwd] {rule} without lambda")
    w, dO, dS, x0, h0 = _problem(rule, "identity", "bf16", 128, 128, 96, True, 5, lam_kind="none",
                                 beta_kind="one" if rule == "additive" else None)
    _compare(*_run(w, dO, dS, x0, h0, "identity", True, with_dS=False))


def test_backward_lone_noop_step():
    """T = 1 with no carried key: the delta rule's step neither decays nor writes, so only
    the read has gradients; the final-state gradient passes straight through."""
    say("[bwd] delta T=1 no carried key")
    w, dO, dS, x0, h0 = _problem("delta", "identity", "f32", 64, 64, 1, False, 9)
    g, ref, _ = _run(w, dO, dS, x0, h0, "identity", False)
    _compare(g, ref, w)
    assert np.all(g["v"].cpu().numpy() == 0) and np.all(g["beta"].cpu().numpy() == 0)


def test_backward_empty_sequence():
    import torch
    say("[bwd] T = 0")
    B, H, d = 2, 3, 128
    dS = np.random.default_rng(3).standard_normal((B, H, d, d)).astype(np.float32)
    gS = make_state(B, H, d, d, S=dS)
    e = torch.empty((B, H, 0, d), dtype=torch.bfloat16, device="cuda")
    g = F.scan_bwd(e, e, e, torch.empty((B, H, 0), device="cuda"), None,
                   torch.empty((B, H, 0, d), device="cuda"), rule=wl.RULE_DELTA, grad_S_out=gS)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(g["state"].S.cpu().numpy(), dS)
    assert np.all(g["state"].x_prev.cpu().numpy() == 0)


def test_backward_is_deterministic():
    """Two calls on the same inputs give bit-identical gradients (no atomics)."""
    say("[bwd] repeatability")
    w, dO, dS, x0, h0 = _problem("delta", "identity", "bf16", 128, 128, 140, True, 11)
    g1 = _run(w, dO, dS, x0, h0, "identity", True)[0]
    g2 = _run(w, dO, dS, x0, h0, "identity", True)[0]
    for n in ("q", "k", "v", "beta", "lam"):
        assert np.array_equal(g1[n].cpu().numpy(), g2[n].cpu().numpy()), n
    assert np.array_equal(g1["state"].buf.cpu().numpy(), g2["state"].buf.cpu().numpy())


@pytest.mark.parametrize("name,heads", [
    ("delta_bf16_h16", [(0, 3), (3, 15)]),   # the benchmark shape, B4 H16 T4096
    ("inner_bf16", [(2, 5)]),                # B4 H8 T4096
    ("additive_bf16", [(1, 9)]),             # B2 H16 T16384, elu+1
])
def test_backward_full_size_sampled_heads(name, heads):
    """The whole workload at its full size through one backward launch, as bench.py
    times it (grad_out ~ N(0,1), no final-state gradient); the oracle then follows a
    few heads on their own (heads are independent), every gradient compared."""
    import torch
    w = wl.SCAN_WORKLOADS[name](seed=0)
    say(f"[bwd full] {name} B={w.B} H={w.H} T={w.T}: oracle on heads {heads}")
    dO = np.random.default_rng(77).standard_normal((w.B, w.H, w.T, w.dv)).astype(np.float32)
    flags = F.PHI_ELU1 if w.phi == wl.PHI_ELU1 else 0
    g = F.scan_bwd(dev_tensor(w.q, w.dtype), dev_tensor(w.k, w.dtype), dev_tensor(w.v, w.dtype),
                   f32_tensor(w.beta), f32_tensor(w.lam), f32_tensor(dO), rule=w.rule,
                   flags=flags, eps=w.eps)
    torch.cuda.synchronize()
    for b, h in heads:
        sl = lambda a: None if a is None else a[b:b + 1, h:h + 1]
        ref = orc.scan_backward(sl(w.q), sl(w.k), sl(w.v), sl(w.beta), sl(w.lam), sl(dO),
                                rule=w.rule, phi_kind=w.phi, eps=w.eps)
        got = {n: None if g[n] is None else g[n][b:b + 1, h:h + 1]
               for n in ("q", "k", "v", "beta", "lam")}
        errs = {}
        for n, x in got.items():
            if ref[n] is None:
                assert x is None, n
                continue
            errs[n] = orc.relerr(x.cpu().numpy().astype(np.float64), ref[n])
        errs["S0"] = orc.relerr(g["state"].S[b:b + 1, h:h + 1].cpu().numpy().astype(np.float64),
                                ref["S0"])
        say(f"    head ({b},{h}): " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
        for n, e in errs.items():
            assert e <= _tol(w), f"grad {n}: {e:.3e}"


@pytest.mark.parametrize("rule,beta_act,per_channel,dtype,T", [
    ("delta", "sigmoid2", False, "bf16", 130),
    ("delta", "sigmoid", True, "f32", 70),
    ("inner", "sigmoid2", False, "bf16", 100),
    ("inner", "sigmoid", True, "bf16", 65),
    ("additive", "sigmoid", False, "bf16", 129),
    ("additive", None, True, "f32", 40),
])
def test_backward_pre_activated_gates(rule, beta_act, per_channel, dtype, T):
    """Gates given as pre-activations (FWMEM_BETA_SIGMOID(2), FWMEM_LAMBDA_PREACT): the
    library activates them as it stages them, and returns the gradients with respect to
    the pre-activations, against the oracle's scan_backward with the same activations."""
    r = RULES[rule]
    bkind = {"sigmoid": "sigmoid", "sigmoid2": "two_sigmoid", None: "one"}[beta_act]
    lkind = "gamma" if r == wl.RULE_ADDITIVE else "softplus"
    say(f"[bwd gates] {rule} beta={beta_act} pc={per_channel} {dtype} T={T}")
    w = wl.make_scan(B=2, H=2, T=T, dk=128, dv=64, dtype=dtype, rule=r, beta_kind=bkind,
                     lam_kind=lkind, lam_mu=-3.0, per_channel=per_channel, s0_std=0.1,
                     seed=T + 3 * per_channel)
    rng = np.random.default_rng(T)
    dO = rng.standard_normal((w.B, w.H, T, w.dv)).astype(np.float32)
    dS = (rng.standard_normal((w.B, w.H, w.dk, w.dv)) * 0.3).astype(np.float32)
    flags = (F.LAMBDA_PREACT | (F.LAMBDA_PER_CHANNEL if per_channel else 0)
             | {"sigmoid": F.BETA_SIGMOID, "sigmoid2": F.BETA_SIGMOID2, None: 0}[beta_act])
    S_in = make_state(w.B, w.H, w.dk, w.dv, S=w.S0)
    g = F.scan_bwd(dev_tensor(w.q, w.dtype), dev_tensor(w.k, w.dtype), dev_tensor(w.v, w.dtype),
                   f32_tensor(w.beta_pre), f32_tensor(w.lam_pre), f32_tensor(dO), rule=r,
                   flags=flags, eps=w.eps, S_in=S_in, grad_S_out=make_state(w.B, w.H, w.dk, w.dv, S=dS))
    ref = orc.scan_backward(w.q, w.k, w.v, w.beta_pre, w.lam_pre, dO, dS, rule=r, eps=w.eps,
                            per_channel=per_channel, S0=w.S0, beta_act=beta_act, lam_act=True)
    _compare(g, ref, w)


@pytest.mark.parametrize("rule,qk,dtype,dk,dv,T,per_channel", [
    ("delta", "l2", "bf16", 128, 128, 130, False),
    ("delta", "rms", "f32", 64, 128, 70, True),
    ("inner", "rms", "bf16", 128, 64, 100, False),
    ("inner", "l2", "f32", 64, 64, 65, False),
    ("additive", "l2", "bf16", 128, 128, 129, False),
    ("additive", "rms", "f32", 64, 64, 40, True),
])
def test_backward_qk_norm(rule, qk, dtype, dk, dv, T, per_channel):
    """Raw q, k and a raw carried key, rescaled by the library (FWMEM_QK_L2NORM /
    FWMEM_QK_RMSNORM): gradients with respect to the raw vectors against the oracle's
    scan_backward with the same qk_norm."""
    r = RULES[rule]
    say(f"[bwd qk] {rule} {qk} {dtype} dk={dk} dv={dv} T={T} pc={per_channel}")
    w = wl.make_scan(B=2, H=2, T=T, dk=dk, dv=dv, dtype=dtype, rule=r,
                     beta_kind="sigmoid" if r == wl.RULE_ADDITIVE else "two_sigmoid",
                     lam_kind="gamma" if r == wl.RULE_ADDITIVE else "softplus", lam_mu=-3.0,
                     per_channel=per_channel, normalise_qk=False, qk_norm=qk, s0_std=0.1,
                     seed=T + dk)
    rng = np.random.default_rng(T + 1)
    x0 = (rng.standard_normal((w.B, w.H, dk)) * 3).astype(np.float32)   # a raw carried key
    h0 = np.ones((w.B, w.H), np.int32)
    dO = rng.standard_normal((w.B, w.H, T, dv)).astype(np.float32)
    dS = (rng.standard_normal((w.B, w.H, dk, dv)) * 0.3).astype(np.float32)
    flags = ({"l2": F.QK_L2NORM, "rms": F.QK_RMSNORM}[qk]
             | (F.LAMBDA_PER_CHANNEL if per_channel else 0))
    g = F.scan_bwd(dev_tensor(w.q, w.dtype), dev_tensor(w.k, w.dtype), dev_tensor(w.v, w.dtype),
                   f32_tensor(w.beta), f32_tensor(w.lam), f32_tensor(dO), rule=r, flags=flags,
                   eps=w.eps, S_in=make_state(w.B, w.H, dk, dv, S=w.S0, xprev=x0, has=h0),
                   grad_S_out=make_state(w.B, w.H, dk, dv, S=dS))
    ref = orc.scan_backward(w.q, w.k, w.v, w.beta, w.lam, dO, dS, rule=r, eps=w.eps,
                            per_channel=per_channel, S0=w.S0, xprev0=x0, has0=h0, qk_norm=qk)
    _compare(g, ref, w)


@pytest.mark.parametrize("rule,dtype,dk,dv,T,extra", [
    ("delta", "bf16", 128, 128, 130, None),
    ("delta", "f32", 64, 128, 70, "qk_gates"),
    ("inner", "bf16", 128, 64, 100, None),
    ("inner", "f32", 64, 64, 65, "qk_gates"),
])
def test_backward_scaled_ridge(rule, dtype, dk, dv, T, extra):
    """The scale-coupled ridge (FWMEM_LAMBDA_SCALED, lambda |x|^2, scalar lambda), alone
    and with RMS normalisation of raw q, k and pre-activated gates, against the oracle's
    scan_backward with the same options."""
    r = RULES[rule]
    both = extra == "qk_gates"
    say(f"[bwd scaled] {rule} {dtype} dk={dk} dv={dv} T={T} extra={extra}")
    w = wl.make_scan(B=2, H=2, T=T, dk=dk, dv=dv, dtype=dtype, rule=r, beta_kind="two_sigmoid",
                     lam_kind="softplus", lam_mu=-3.0, normalise_qk=not both,
                     qk_norm="rms" if both else None, s0_std=0.1, seed=T + 7)
    rng = np.random.default_rng(T + 2)
    x0 = (rng.standard_normal((w.B, w.H, dk)) * (3 if both else 0.09)).astype(np.float32)
    h0 = np.ones((w.B, w.H), np.int32)
    dO = rng.standard_normal((w.B, w.H, T, dv)).astype(np.float32)
    dS = (rng.standard_normal((w.B, w.H, dk, dv)) * 0.3).astype(np.float32)
    flags = F.LAMBDA_SCALED | ((F.QK_RMSNORM | F.BETA_SIGMOID2 | F.LAMBDA_PREACT) if both else 0)
    beta = w.beta_pre if both else w.beta
    lam = w.lam_pre if both else w.lam
    g = F.scan_bwd(dev_tensor(w.q, w.dtype), dev_tensor(w.k, w.dtype), dev_tensor(w.v, w.dtype),
                   f32_tensor(beta), f32_tensor(lam), f32_tensor(dO), rule=r, flags=flags, eps=w.eps,
                   S_in=make_state(w.B, w.H, dk, dv, S=w.S0, xprev=x0, has=h0),
                   grad_S_out=make_state(w.B, w.H, dk, dv, S=dS))
    ref = orc.scan_backward(w.q, w.k, w.v, beta, lam, dO, dS, rule=r, eps=w.eps, S0=w.S0,
                            xprev0=x0, has0=h0, lam_scaled=True,
                            qk_norm="rms" if both else None,
                            beta_act="sigmoid2" if both else None, lam_act=both)
    _compare(g, ref, w)


@pytest.mark.parametrize("dtype,dk,dv,T,extra", [
    ("bf16", 128, 128, 130, None),
    ("f32", 64, 128, 70, "elu1"),
    ("bf16", 128, 64, 97, "rms_scaled_gates"),
    ("f32", 64, 64, 33, None),
])
def test_backward_per_value_channel(dtype, dk, dv, T, extra):
    """FWMEM_RULE_DELTA_PV: beta [B,H,T,dv], one step size and decay per value column;
    every gradient (beta's per column) against the oracle's scan_backward, plain, with
    elu+1, and with RMS normalisation, the scale-coupled ridge and pre-activated gates."""
    r = wl.RULE_DELTA_PV
    opts = extra == "rms_scaled_gates"
    phi = "elu1" if extra == "elu1" else "identity"
    say(f"[bwd pv] {dtype} dk={dk} dv={dv} T={T} extra={extra}")
    w = wl.make_scan(B=2, H=2, T=T, dk=dk, dv=dv, dtype=dtype, rule=r, beta_kind="two_sigmoid",
                     lam_kind="softplus", lam_mu=-3.0,
                     phi=wl.PHI_ELU1 if phi == "elu1" else wl.PHI_IDENTITY,
                     normalise_qk=not opts and phi != "elu1", qk_norm="rms" if opts else None,
                     s0_std=0.1, seed=T + dv)
    rng = np.random.default_rng(T + 3)
    kp = rng.standard_normal((w.B, w.H, dk)).astype(np.float32)
    x0 = (kp * 3 if opts else kp / np.linalg.norm(kp, axis=-1, keepdims=True)).astype(np.float32)
    if phi == "elu1":
        x0 = np.where(x0 > 0, x0 + 1.0, np.exp(x0)).astype(np.float32)
    h0 = np.ones((w.B, w.H), np.int32)
    dO = rng.standard_normal((w.B, w.H, T, dv)).astype(np.float32)
    dS = (rng.standard_normal((w.B, w.H, dk, dv)) * 0.3).astype(np.float32)
    flags = ((F.PHI_ELU1 if phi == "elu1" else 0)
             | ((F.QK_RMSNORM | F.LAMBDA_SCALED | F.BETA_SIGMOID2 | F.LAMBDA_PREACT) if opts else 0))
    beta = w.beta_pre if opts else w.beta
    lam = w.lam_pre if opts else w.lam
    g = F.scan_bwd(dev_tensor(w.q, w.dtype), dev_tensor(w.k, w.dtype), dev_tensor(w.v, w.dtype),
                   f32_tensor(beta), f32_tensor(lam), f32_tensor(dO), rule=r, flags=flags, eps=w.eps,
                   S_in=make_state(w.B, w.H, dk, dv, S=w.S0, xprev=x0, has=h0),
                   grad_S_out=make_state(w.B, w.H, dk, dv, S=dS))
    assert tuple(g["beta"].shape) == (w.B, w.H, T, dv)
    ref = orc.scan_backward(w.q, w.k, w.v, beta, lam, dO, dS, rule=r, phi_kind=phi, eps=w.eps,
                            S0=w.S0, xprev0=x0, has0=h0, qk_norm="rms" if opts else None,
                            lam_scaled=opts, beta_act="sigmoid2" if opts else None, lam_act=opts)
    _compare(g, ref, w)


@pytest.mark.parametrize("phi,dtype,dk,dv,T,extra", [
    ("identity", "bf16", 128, 128, 130, None),
    ("elu1", "f32", 64, 128, 70, None),
    ("identity", "bf16", 128, 64, 97, "qk_gates"),
    ("elu1", "bf16", 64, 64, 33, None),
])
def test_backward_normaliser(phi, dtype, dk, dv, T, extra):
    """Normalised linear attention (FWMEM_ZNORM, additive rule): o = S^T q / (z.q + eps).
    Every gradient, the initial z's (the carried-key slot) included, against the oracle's
    scan_backward, from a nonzero S0 and z0; positive features keep z.q away from zero."""
    r = wl.RULE_ADDITIVE
    both = extra == "qk_gates"
    say(f"[bwd znorm] {phi} {dtype} dk={dk} dv={dv} T={T} extra={extra}")
    w = wl.make_scan(B=2, H=2, T=T, dk=dk, dv=dv, dtype=dtype, rule=r, beta_kind="sigmoid",
                     lam_kind="gamma", phi=wl.PHI_ELU1 if phi == "elu1" else wl.PHI_IDENTITY,
                     normalise_qk=phi != "elu1" and not both, qk_positive=phi != "elu1",
                     qk_norm="l2" if both else None, znorm=True, s0_std=0.05, seed=T + dk)
    rng = np.random.default_rng(T + 5)
    dO = rng.standard_normal((w.B, w.H, T, dv)).astype(np.float32)
    dS = (rng.standard_normal((w.B, w.H, dk, dv)) * 0.3).astype(np.float32)
    dz = (rng.standard_normal((w.B, w.H, dk)) * 0.3).astype(np.float32)  # the final z's gradient
    flags = (F.ZNORM | (F.PHI_ELU1 if phi == "elu1" else 0)
             | ((F.QK_L2NORM | F.BETA_SIGMOID | F.LAMBDA_PREACT) if both else 0))
    beta = w.beta_pre if both else w.beta
    lam = w.lam_pre if both else w.lam
    g = F.scan_bwd(dev_tensor(w.q, w.dtype), dev_tensor(w.k, w.dtype), dev_tensor(w.v, w.dtype),
                   f32_tensor(beta), f32_tensor(lam), f32_tensor(dO), rule=r, flags=flags, eps=w.eps,
                   S_in=make_state(w.B, w.H, dk, dv, S=w.S0, xprev=w.xprev0),
                   grad_S_out=make_state(w.B, w.H, dk, dv, S=dS, xprev=dz))
    ref = orc.scan_backward(w.q, w.k, w.v, beta, lam, dO, dS, rule=r, phi_kind=phi, eps=w.eps,
                            S0=w.S0, xprev0=w.xprev0, znorm=True, qk_norm="l2" if both else None,
                            beta_act="sigmoid" if both else None, lam_act=both, dz=dz)
    assert np.any(ref["xprev0"] != 0)
    _compare(g, ref, w)


def test_backward_normaliser_chains_over_calls():
    """A normalised linear-attention sequence split over two calls: the backward of the
    second call (from the first call's final state), then the backward of the first call
    with the second's grad_S_in as its grad_S_out (the S part and the normaliser's
    gradient in the x_prev part), gives the gradients of one call over the whole
    sequence. fp32 inputs, so that the forward state handed between the calls is as
    exact as the backward's own recomputation."""
    r, dk, dv, T, T1 = wl.RULE_ADDITIVE, 64, 128, 150, 70
    w = wl.make_scan(B=2, H=2, T=T, dk=dk, dv=dv, dtype="f32", rule=r, beta_kind="sigmoid",
                     lam_kind="gamma", phi=wl.PHI_ELU1, normalise_qk=False, znorm=True,
                     s0_std=0.05, seed=11)
    rng = np.random.default_rng(12)
    dO = rng.standard_normal((w.B, w.H, T, dv)).astype(np.float32)
    dS = (rng.standard_normal((w.B, w.H, dk, dv)) * 0.3).astype(np.float32)
    dz = (rng.standard_normal((w.B, w.H, dk)) * 0.3).astype(np.float32)
    flags = F.ZNORM | F.PHI_ELU1
    dev = lambda x, a, e: dev_tensor(np.ascontiguousarray(x[:, :, a:e]), "f32")
    S0 = lambda: make_state(w.B, w.H, dk, dv, S=w.S0, xprev=w.xprev0)
    say("[bwd znorm chain] one call")
    g = F.scan_bwd(dev(w.q, 0, T), dev(w.k, 0, T), dev(w.v, 0, T), dev(w.beta, 0, T),
                   dev(w.lam, 0, T), dev(dO, 0, T), rule=r, flags=flags, eps=w.eps, S_in=S0(),
                   grad_S_out=make_state(w.B, w.H, dk, dv, S=dS, xprev=dz))
    say("[bwd znorm chain] forward of the first part, then the two backward calls")
    _, S1 = F.scan_fwd(dev(w.q, 0, T1), dev(w.k, 0, T1), dev(w.v, 0, T1), dev(w.beta, 0, T1),
                       dev(w.lam, 0, T1), rule=r, flags=flags, eps=w.eps, S_in=S0())
    g2 = F.scan_bwd(dev(w.q, T1, T), dev(w.k, T1, T), dev(w.v, T1, T), dev(w.beta, T1, T),
                    dev(w.lam, T1, T), dev(dO, T1, T), rule=r, flags=flags, eps=w.eps, S_in=S1,
                    grad_S_out=make_state(w.B, w.H, dk, dv, S=dS, xprev=dz))
    g1 = F.scan_bwd(dev(w.q, 0, T1), dev(w.k, 0, T1), dev(w.v, 0, T1), dev(w.beta, 0, T1),
                    dev(w.lam, 0, T1), dev(dO, 0, T1), rule=r, flags=flags, eps=w.eps, S_in=S0(),
                    grad_S_out=g2["state"])
    ref = orc.scan_backward(w.q, w.k, w.v, w.beta, w.lam, dO, dS, rule=r, phi_kind="elu1",
                            eps=w.eps, S0=w.S0, xprev0=w.xprev0, znorm=True, dz=dz)
    _compare(g, ref, w)
    for name in ("q", "k", "v", "beta", "lam"):
        both_parts = np.concatenate([g1[name].cpu().numpy(), g2[name].cpu().numpy()], axis=2)
        e = orc.relerr(both_parts, g[name].cpu().numpy())
        assert e <= TOL["f32"], (name, e)
    for name in ("S", "x_prev"):
        e = orc.relerr(getattr(g1["state"], name).cpu().numpy(), getattr(g["state"], name).cpu().numpy())
        assert e <= TOL["f32"], (name, e)
