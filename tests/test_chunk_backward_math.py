"""The chunk-parallel form of the scan's backward pass, run in float64 on the CPU and
matched against the oracle's token-serial scan_backward (reading D21).

The GPU's chunked backward computes exactly these steps; this test checks the algebra
itself, independently of the kernels. Per head, with chunks of C tokens and, inside a
chunk, Gamma_t the product of the decays a_s (s <= t), Gamma_end the chunk's total,
D_ts = Gamma_t / Gamma_s (s <= t) and D'_ts = Gamma_{t-1} / Gamma_s (s < t):

  forward (entry state S, exit S'):
    L = diag(eta) (D' o X X^T),  T = (I + L)^-1,  M = D o (Q X^T)
    U = T diag(eta) (V - diag(Gamma_prev) X S)      (delta rule)
    U = diag(f) V                                   (inner: f = eta; additive: f = beta)
    O = diag(Gamma) Q S + M U,   S' = Gamma_end S + X^T diag(Gamma_end / Gamma) U
  backward, serial over chunks from the last (dS' the exit gradient, dO the chunk's):
    dU = M^T dO + diag(Gamma_end / Gamma) X dS',   dR = T^T dU
    dS = Gamma_end dS' + Q^T diag(Gamma) dO - X^T diag(eta Gamma_prev) dR
  then per chunk, in parallel, the gradients of Q, X, V, eta (or f) and of the log
  decays from the stored entry state S and exit gradient dS'.
"""
import numpy as np
import pytest

from oracle import fwmem_oracle as orc

DELTA, ADD, INNER = orc.RULE_DELTA, orc.RULE_ADDITIVE, orc.RULE_INNER


def _phi(x, kind):
    return np.where(x > 0, x + 1.0, np.exp(x)) if kind == "elu1" else x


def _dphi(x, kind):
    return np.where(x > 0, 1.0, np.exp(x)) if kind == "elu1" else np.ones_like(x)


def chunked_backward(q, k, v, beta, lam, dO, dS, *, rule, phi_kind, eps, C, S0, x0, has0,
                     lam_scaled=False):
    """One head: q, k [T, dk], v [T, dv], beta/lam [T] (or None), dO [T, dv], dS [dk, dv].
    Returns the gradients of q, k, v, beta, lam, S0 and the carried key."""
    T, dk = q.shape
    dv = v.shape[1]
    nlms = rule != ADD
    qt, kt = _phi(q, phi_kind), _phi(k, phi_kind)
    # per-token written key, step size (or write scale) and decay
    X = np.zeros((T, dk))
    key = np.zeros(T, dtype=bool)
    eta, a, den, lam_used, nn = np.zeros(T), np.ones(T), np.ones(T), np.zeros(T), np.zeros(T)
    for t in range(T):
        if nlms:
            if t >= 1:
                X[t], key[t] = kt[t - 1], True
            elif has0:
                X[t], key[t] = x0, True
            if key[t]:
                nn[t] = X[t] @ X[t]
                lt = 0.0 if lam is None else lam[t]
                lam_used[t] = lt * nn[t] if lam_scaled else lt
                den[t] = nn[t] + lam_used[t] + eps
                eta[t] = beta[t] / den[t]
                a[t] = 1.0 - eta[t] * lam_used[t]
        else:
            X[t], key[t] = kt[t], True
            eta[t] = 1.0 if beta is None else beta[t]
            a[t] = 1.0 if lam is None else lam[t]
    nch = (T + C - 1) // C

    def chunk(c):
        t0, t1 = c * C, min(T, c * C + C)
        n = t1 - t0
        pad = lambda z: np.concatenate([z[t0:t1], np.zeros((C - n,) + z.shape[1:])])
        Xc, Qc, Vc, dOc = pad(X), pad(qt), pad(v), pad(dO)
        Ec = pad(eta)
        Ac = np.concatenate([a[t0:t1], np.ones(C - n)])
        Gam = np.cumprod(Ac)
        Gprev = np.concatenate([[1.0], Gam[:-1]])
        Gend = Gam[-1]
        D = np.tril(Gam[:, None] / Gam[None, :])
        Dp = np.tril(Gprev[:, None] / Gam[None, :], -1)
        Gx = Xc @ Xc.T
        M = D * (Qc @ Xc.T)
        L = Ec[:, None] * Dp * Gx
        Tm = np.linalg.inv(np.eye(C) + L)
        return dict(t0=t0, t1=t1, n=n, X=Xc, Q=Qc, V=Vc, dO=dOc, E=Ec, A=Ac, Gam=Gam,
                    Gprev=Gprev, Gend=Gend, D=D, Dp=Dp, Gx=Gx, M=M, L=L, Tm=Tm)

    def write(ch, S):
        if rule == DELTA:
            Rhat = ch["V"] - ch["Gprev"][:, None] * (ch["X"] @ S)
            return ch["Tm"] @ (ch["E"][:, None] * Rhat), Rhat
        return ch["E"][:, None] * ch["V"], None

    # forward: the state at every chunk start
    Sc = [S0.copy()]
    for c in range(nch):
        ch = chunk(c)
        U, _ = write(ch, Sc[-1])
        Sc.append(ch["Gend"] * Sc[-1] + ch["X"].T @ ((ch["Gend"] / ch["Gam"])[:, None] * U))

    # backward chain: the exit gradient of every chunk
    dSx = [None] * nch
    G = dS.copy()
    for c in range(nch - 1, -1, -1):
        ch = chunk(c)
        dSx[c] = G
        dU = ch["M"].T @ ch["dO"] + (ch["Gend"] / ch["Gam"])[:, None] * (ch["X"] @ G)
        Gn = ch["Gend"] * G + ch["Q"].T @ (ch["Gam"][:, None] * ch["dO"])
        if rule == DELTA:
            dR = ch["Tm"].T @ dU
            Gn = Gn - ch["X"].T @ ((ch["E"] * ch["Gprev"])[:, None] * dR)
        G = Gn
    dS0 = G

    # per chunk gradients
    gq, gX, gv = np.zeros((T, dk)), np.zeros((T, dk)), np.zeros((T, dv))
    deta, dl = np.zeros(T), np.zeros(T)
    for c in range(nch):
        ch = chunk(c)
        S, dSp = Sc[c], dSx[c]
        Xc, Q, V, dOc, E = ch["X"], ch["Q"], ch["V"], ch["dO"], ch["E"]
        Gam, Gprev, Gend, D, Dp = ch["Gam"], ch["Gprev"], ch["Gend"], ch["D"], ch["Dp"]
        U, Rhat = write(ch, S)
        dU = ch["M"].T @ dOc + (Gend / Gam)[:, None] * (Xc @ dSp)
        dQ1 = Gam[:, None] * (dOc @ S.T)
        dMm = np.tril(dOc @ U.T)
        dQ = dQ1 + (dMm * D) @ Xc
        dXS = (Gend / Gam)[:, None] * (U @ dSp.T)
        dX = (dMm * D).T @ Q + dXS
        dg = np.sum(Q * dQ1, axis=1)
        PM = dMm * ch["M"]
        dg += PM.sum(axis=1) - PM.sum(axis=0)
        h = np.sum(Xc * dXS, axis=1)
        dg -= h
        dg[C - 1] += h.sum() + Gend * np.sum(dSp * S)
        if rule == DELTA:
            dR = ch["Tm"].T @ dU
            dVc = E[:, None] * dR
            dXR = -(E * Gprev)[:, None] * (dR @ S.T)
            dX += dXR
            dg[:-1] += np.sum(Xc * dXR, axis=1)[1:]
            dLm = np.tril(-dR @ U.T, -1)
            W = dLm * E[:, None] * Dp
            dX += W @ Xc + W.T @ Xc
            PL = dLm * ch["L"]
            dg[:-1] += PL.sum(axis=1)[1:]
            dg -= PL.sum(axis=0)
            de = np.sum(dR * Rhat, axis=1) + np.sum(dLm * Dp * ch["Gx"], axis=1)
        else:
            dVc = E[:, None] * dU
            de = np.sum(dU * V, axis=1)
        dlc = np.cumsum(dg[::-1])[::-1]
        t0, t1, n = ch["t0"], ch["t1"], ch["n"]
        gq[t0:t1] = dQ[:n]
        gX[t0:t1] = dX[:n]
        gv[t0:t1] = dVc[:n]
        deta[t0:t1] = de[:n]
        dl[t0:t1] = dlc[:n]

    da = dl / a
    gbeta = None if beta is None else np.zeros(T)
    glam = None if lam is None else np.zeros(T)
    for t in range(T):
        if not key[t]:
            continue
        if nlms:
            de = deta[t] - lam_used[t] * da[t]
            gbeta[t] = de / den[t]
            dden = -eta[t] * de / den[t]
            dlu = -eta[t] * da[t] + dden
            dn = dden + (lam[t] * dlu if (lam_scaled and lam is not None) else 0.0)
            if glam is not None:
                glam[t] = dlu * (nn[t] if lam_scaled else 1.0)
            gX[t] += 2.0 * dn * X[t]
        else:
            if gbeta is not None:
                gbeta[t] = deta[t]
            if glam is not None:
                glam[t] = da[t]
    gk = np.zeros((T, dk))
    gx0 = np.zeros(dk)
    if nlms:
        gk[:-1] = gX[1:] * _dphi(k[:-1], phi_kind)
        if has0:
            gx0 = gX[0]
    else:
        gk = gX * _dphi(k, phi_kind)
    return dict(q=gq * _dphi(q, phi_kind), k=gk, v=gv, beta=gbeta, lam=glam, S0=dS0, xprev0=gx0)


@pytest.mark.parametrize("rule,phi_kind,T,C,carried,lam_scaled", [
    (DELTA, "identity", 37, 8, True, False),
    (DELTA, "identity", 32, 8, False, False),
    (DELTA, "elu1", 29, 16, True, False),
    (DELTA, "identity", 40, 16, True, True),
    (INNER, "identity", 37, 8, True, False),
    (INNER, "elu1", 24, 8, False, True),
    (ADD, "identity", 37, 8, True, False),
    (ADD, "elu1", 19, 8, False, False),
])
def test_chunked_backward_equals_the_token_serial_oracle(rule, phi_kind, T, C, carried, lam_scaled):
    rng = np.random.default_rng(T * 7 + C + rule)
    dk, dv = 6, 5
    q, k, v = (rng.standard_normal((T, d)) for d in (dk, dk, dv))
    if phi_kind == "identity":
        q /= np.linalg.norm(q, axis=1, keepdims=True)
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    beta = rng.uniform(0.1, 1.9, T)
    lam = rng.uniform(0.6, 1.0, T) if rule == ADD else rng.uniform(0.01, 0.4, T)
    dO, dS = rng.standard_normal((T, dv)), rng.standard_normal((dk, dv))
    S0 = rng.standard_normal((dk, dv)) * 0.3 if carried else np.zeros((dk, dv))
    x0 = _phi(rng.standard_normal(dk) * 0.5, phi_kind)
    has0 = carried and rule != ADD
    got = chunked_backward(q, k, v, beta, lam, dO, dS, rule=rule, phi_kind=phi_kind, eps=1e-6,
                           C=C, S0=S0, x0=x0, has0=has0, lam_scaled=lam_scaled)
    e4 = lambda z: z[None, None]
    ref = orc.scan_backward(e4(q), e4(k), e4(v), e4(beta), e4(lam), e4(dO), e4(dS), rule=rule,
                            phi_kind=phi_kind, eps=1e-6, S0=e4(S0), lam_scaled=lam_scaled,
                            xprev0=e4(x0) if has0 else None,
                            has0=np.array([[1]]) if has0 else None)
    for name in ("q", "k", "v", "beta", "lam", "S0", "xprev0"):
        np.testing.assert_allclose(got[name], ref[name][0, 0], rtol=1e-9, atol=1e-10, err_msg=name)
