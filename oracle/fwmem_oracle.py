"""Plain fp64 CPU oracle for the fast-weight matrix-memory scan.

TEST INFRASTRUCTURE. Only tests/, the smoke check and the benchmark's CPU
baseline leg may import or run this module. The library never calls it, and it
shares no code with the HIP path (it imports nothing from that package).

It is the sequential recurrence written out, one token at a time, in float64,
vectorised only over independent heads (b, h). Sources (page titles as printed):

  [FWA]  "Fast Weight Attention for Continual Learning" reading notes
         (inkeast.github.io MessageDaily): section 3.2 (instantaneous ridge loss and
         its normalised gradient step), section 4.1 (read-after-write pairing
         x_t = phi(k_{t-1}), y_t = v_t and the boundary x_1 = 0, eta_1 = 0),
         section 4.2 (Falcon-1 rule, beta in (0,2), per-step descent lemma,
         NLMS limit), section 4.3 (the inner-product family, Falcon-1A: the same
         shifted pair, step size and decay, with the target written in place of the
         residual), section 4.4 (Falcon-2: the squared error separates over the value
         channels, so each channel takes its own step size with the shared pair),
         section 4.5 (RMSNorm of q and k; the ridge coupled to an energy
         statistic so that the decay does not depend on the input scale).
  [AFFN] hncyxsy.com blog post "attention is also an FFN" (news/211194):
         section 2.1 (S_i = sum_{j<=i} phi(k_j) v_j^T, y_i = phi(q_i)^T S_i),
         section 3.2 (decayed write S_t = lambda S_{t-1} + phi(k_t) v_t^T),
         section 4.1 (phi = elu + 1, state of shape d_k x d_v kept in fp32).

Readings where the pages leave a step open (listed in the design doc as D1..D14):
  D1  per-key-channel lambda: the decay is diag(1 - eta*lambda_t) on the rows of S
      and eta's denominator uses max_i lambda_{t,i}.
  D2  step 1 of a sequence (no previous key) neither decays nor writes.
  D3  the shifted key crosses call boundaries through (xprev, has_prev).
  D4  beta_t, lambda_t are indexed by the target's step t.
  D7  additive rule: the `lam` slot carries the retention gamma_t (None = 1) and
      `beta` an optional write scale (None = 1); pairing is same-index.
  D16 normalised q and k (qk_norm): each is rescaled to length 1 (l2) or sqrt(d_k)
      (RMSNorm with unit gain and no epsilon), a zero vector stays zero, and the
      carried key is stored raw.
  D17 gate pre-activations (beta_act, lam_act): beta = sigmoid(z) or 2 sigmoid(z); the
      ridge lambda = softplus(z), the additive retention gamma = sigmoid(z).
  D18 normalised linear attention (znorm): o_t = S_t^T phi(q_t) / (z_t . phi(q_t) + eps)
      with z decayed like S; z is carried in the carried-key slot of the state.
  D19 scale-coupled ridge (lam_scaled): lambda_t = lambda_bar_t * ||x_t||^2, the energy
      of the key written at step t (after any normalisation), for every channel of a
      per-channel lambda.
  D20 per-value-channel rule (Falcon-2): beta is [B,H,T,d_v], lambda a scalar per token;
      channel j steps by eta_{j,t} = beta_{j,t} / (|x_t|^2 + lambda_t + eps) and decays
      its own column of S by 1 - eta_{j,t} lambda_t; shifted pair and boundary as D2.
  D21 backward pass (scan_backward): the pages give none; gradients are the reverse-mode
      derivative of the recurrence as the forward pass states it, with lambda-hat's
      maximum passing its gradient to the first channel attaining it.
  D15 inner-product rule: the delta rule's shifted pair, eta_t (with D1 for a
      per-channel lambda), decay 1 - eta_t lambda_t and boundary D2; beta is
      required as for the delta rule.
"""
from __future__ import annotations

import numpy as np

RULE_DELTA = 0
RULE_ADDITIVE = 1
RULE_INNER = 2
RULE_DELTA_PV = 3


def phi(x: np.ndarray, kind: str) -> np.ndarray:
    """Feature map. 'elu1' is elu(x) + 1, i.e. x + 1 for x > 0 and exp(x) otherwise
    ([AFFN] section 4.1); 'identity' returns x."""
    x = np.asarray(x, dtype=np.float64)
    if kind == "identity":
        return x.copy()
    if kind == "elu1":
        return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))
    raise ValueError(kind)


def _heads(a, tail_ndim):
    """Flatten leading (B, H) into one head axis."""
    a = np.asarray(a, dtype=np.float64)
    return a.reshape((-1,) + a.shape[a.ndim - tail_ndim:])


def sigmoid(z: np.ndarray) -> np.ndarray:
    """1 / (1 + e^-z), in float64."""
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def softplus(z: np.ndarray) -> np.ndarray:
    """log(1 + e^z), in float64 (z itself where e^z would overflow the sum's precision)."""
    z = np.asarray(z, dtype=np.float64)
    return np.where(z > 30.0, z, np.log1p(np.exp(np.minimum(z, 30.0))))


def unit_rows(x: np.ndarray, length: float = 1.0) -> np.ndarray:
    """Each row (last axis) rescaled to the given Euclidean length; a zero row stays
    zero (reading D16)."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.divide(x * length, n, out=np.zeros_like(x), where=n > 0)


def scan(q, k, v, beta, lam, *, rule, phi_kind="identity", eps=1e-6, per_channel=False,
         S0=None, xprev0=None, has0=None, qk_norm=None, beta_act=None, lam_act=False,
         znorm=False, lam_scaled=False):
    """Run the recurrence over a whole sequence.

    q, k: [B,H,T,dk]; v: [B,H,T,dv]; beta: [B,H,T] or None; lam: [B,H,T] (or
    [B,H,T,dk] when per_channel) or None. S0: [B,H,dk,dv] or None (zeros);
    xprev0: [B,H,dk] or None; has0: [B,H] or None (no previous key).
    qk_norm: None, "l2" or "rms". q_t and k_t are used rescaled to unit length ("l2")
    or to root-mean-square 1, i.e. length sqrt(d_k) ("rms": RMSNorm with unit gain).
    [FWA] section 4.5 normalises the query and key projections (RMSNorm by default,
    l2 in the DeltaNet variants); reading D16. Identity feature map only. The carried
    key stays the raw k of the last token and is rescaled where it is used.
    beta_act: None, "sigmoid" or "sigmoid2": beta holds pre-activations z and the step
    size (delta, inner) or write scale (additive) is sigmoid(z) or 2 sigmoid(z), the
    latter spanning the range (0, 2) of [FWA] section 4.2. lam_act: lam holds
    pre-activations; the ridge is softplus(z) (delta, inner) and the retention sigmoid(z)
    (additive). Reading D17.
    znorm: additive rule only. The read is divided by the normaliser,
    o_t = S_t^T phi(q_t) / (z_t . phi(q_t) + eps), z_t = gamma_t z_{t-1} + beta_t phi(k_t)
    ([AFFN] section 4.2, with the decay applied to z as well, as that section suggests).
    z takes the place of the carried key in the state (xprev0 / the returned xprev),
    since the additive rule never reads that key (reading D18).
    lam_scaled: delta and inner rules only. lam (after any activation) is a
    dimensionless base ridge, multiplied by the energy ||x_t||^2 of the key written at
    step t ([FWA] section 4.5; reading D19), so that eta_t lambda_t, the decay, is the
    same for any rescaling of the keys.

    Returns (o [B,H,T,dv], S [B,H,dk,dv], xprev [B,H,dk], has [B,H]) in float64.
    """
    q = np.asarray(q)
    B, H, T, dk = q.shape
    dv = np.asarray(v).shape[-1]
    N = B * H
    Q = _heads(q, 2)
    K = _heads(k, 2)
    V = _heads(v, 2)
    Bt = None if beta is None else _heads(beta, 2 if rule == RULE_DELTA_PV else 1)
    if Bt is not None and beta_act is not None:
        Bt = {"sigmoid": 1.0, "sigmoid2": 2.0}[beta_act] * sigmoid(Bt)
    if lam is None:
        Lm = None
    else:
        Lm = _heads(lam, 2 if per_channel else 1)
        if lam_act:
            Lm = sigmoid(Lm) if rule == RULE_ADDITIVE else softplus(Lm)

    S = np.zeros((N, dk, dv)) if S0 is None else _heads(S0, 2).copy()
    xprev = np.zeros((N, dk)) if xprev0 is None else _heads(xprev0, 1).copy()
    has = np.zeros(N, dtype=bool) if has0 is None else (np.asarray(has0).reshape(N) != 0)
    O = np.zeros((N, T, dv))

    if qk_norm is not None and phi_kind != "identity":
        raise ValueError("qk_norm takes the identity feature map")
    if qk_norm is None:
        unit = lambda a: a
    elif qk_norm in ("l2", "rms"):
        length = 1.0 if qk_norm == "l2" else float(np.sqrt(dk))
        unit = lambda a: unit_rows(a, length)
    else:
        raise ValueError(qk_norm)

    if znorm and rule != RULE_ADDITIVE:
        raise ValueError("znorm takes the additive rule")
    if lam_scaled and rule == RULE_ADDITIVE:
        raise ValueError("lam_scaled takes the delta or inner rule")
    if rule == RULE_DELTA_PV and per_channel:
        raise ValueError("the per-value-channel rule takes a scalar lambda")
    z = xprev.copy() if znorm else None

    for t in range(T):
        qt = unit(phi(Q[:, t], phi_kind))
        k_raw = phi(K[:, t], phi_kind)
        kt = unit(k_raw)
        vt = V[:, t]
        if rule in (RULE_DELTA, RULE_INNER):
            # [FWA] 4.1: the pair written at step t is (phi(k_{t-1}), v_t); with no
            # previous key the pair is (0, v_t) with eta = 0, so nothing happens.
            x = np.where(has[:, None], unit(xprev), 0.0)
            if Lm is None:
                lam_t = np.zeros(N)
                lam_hat = lam_t
            elif per_channel:
                lam_t = Lm[:, t, :]                  # [N, dk]
                lam_hat = lam_t.max(axis=1)          # reading D1
            else:
                lam_t = Lm[:, t]
                lam_hat = lam_t
            if lam_scaled:
                energy = np.sum(x * x, axis=1)
                lam_t = lam_t * (energy[:, None] if per_channel else energy)
                lam_hat = lam_hat * energy
            # [FWA] 3.2 / 4.2: eta_t = beta_t / (||x_t||^2 + lambda_t + eps).
            den = np.sum(x * x, axis=1) + lam_hat + eps
            eta = np.where(has, Bt[:, t] / np.where(has, den, 1.0), 0.0)
            decay = 1.0 - (eta[:, None] * lam_t if per_channel else (eta * lam_t)[:, None])
            if rule == RULE_DELTA:
                # residual against the state before this step's write
                r = vt - np.einsum("nij,ni->nj", S, x)
                S = decay[:, :, None] * S + eta[:, None, None] * x[:, :, None] * r[:, None, :]
            else:
                # [FWA] 4.3: the negative inner-product loss -<S^T x_t, y_t> +
                # (lambda_t/2)|S|^2 has gradient lambda_t S - x_t y_t^T, so the step
                # writes the target y_t = v_t itself, with no residual.
                S = decay[:, :, None] * S + eta[:, None, None] * x[:, :, None] * vt[:, None, :]
        elif rule == RULE_DELTA_PV:
            # [FWA] 4.4, Falcon-2: value channel j minimises its own squared error with
            # its own step eta_{j,t} on the shared pair (x_t, v_t), so the rule is d_v
            # scalar-step delta rules side by side, each decaying its own column of S
            # (reading D20).
            x = unit(xprev) * has[:, None]
            lam_pv = np.zeros(N) if Lm is None else Lm[:, t]
            if lam_scaled:
                lam_pv = lam_pv * np.sum(x * x, axis=1)
            den_pv = np.sum(x * x, axis=1) + lam_pv + eps
            eta_pv = np.where(has[:, None], Bt[:, t, :] / np.where(has, den_pv, 1.0)[:, None], 0.0)
            r_pv = vt - np.einsum("ni,nij->nj", x, S)
            S = (1.0 - eta_pv * lam_pv[:, None])[:, None, :] * S + x[:, :, None] * (eta_pv * r_pv)[:, None, :]
        elif rule == RULE_ADDITIVE:
            # [AFFN] 3.2: S_t = gamma_t S_{t-1} + phi(k_t) v_t^T (times an optional
            # write scale beta_t, reading D7).
            if Lm is None:
                gam = np.ones((N, 1, 1))
            elif per_channel:
                gam = Lm[:, t, :, None]
            else:
                gam = Lm[:, t][:, None, None]
            b = np.ones(N) if Bt is None else Bt[:, t]
            S = gam * S + b[:, None, None] * kt[:, :, None] * vt[:, None, :]
            if znorm:
                z = gam[:, :, 0] * z + b[:, None] * kt
        else:
            raise ValueError(rule)
        xprev = z if znorm else k_raw
        has = np.ones(N, dtype=bool)
        # read after write: o_t = S_t^T phi(q_t) ([AFFN] 2.1; [FWA] 4.1)
        O[:, t] = np.einsum("nij,ni->nj", S, qt)
        if znorm:
            O[:, t] /= (np.sum(z * qt, axis=1) + eps)[:, None]

    return (O.reshape(B, H, T, dv), S.reshape(B, H, dk, dv), xprev.reshape(B, H, dk),
            has.reshape(B, H).astype(np.int32))


def step(q, k, v, beta, lam, *, rule, phi_kind="identity", eps=1e-6, per_channel=False,
         S0=None, xprev0=None, has0=None, qk_norm=None, beta_act=None, lam_act=False,
         znorm=False, lam_scaled=False):
    """One-token recurrent decode: q, k: [B,H,dk], v: [B,H,dv], beta/lam: [B,H]
    (lam [B,H,dk] when per_channel; beta [B,H,dv] for the per-value-channel rule).
    Returns (o [B,H,dv], S, xprev, has)."""
    q = np.asarray(q)[:, :, None]
    k = np.asarray(k)[:, :, None]
    v = np.asarray(v)[:, :, None]
    beta = None if beta is None else np.asarray(beta)[:, :, None]
    if lam is not None:
        lam = np.asarray(lam)
        lam = lam[:, :, None, :] if per_channel else lam[:, :, None]
    o, S, xp, h = scan(q, k, v, beta, lam, rule=rule, phi_kind=phi_kind, eps=eps,
                       per_channel=per_channel, S0=S0, xprev0=xprev0, has0=has0, qk_norm=qk_norm,
                       beta_act=beta_act, lam_act=lam_act, znorm=znorm, lam_scaled=lam_scaled)
    return o[:, :, 0], S, xp, h


def phi_grad(x: np.ndarray, kind: str) -> np.ndarray:
    """Derivative of the feature map: 1 for the identity; for elu+1, 1 where x > 0 and
    exp(x) elsewhere."""
    x = np.asarray(x, dtype=np.float64)
    if kind == "identity":
        return np.ones_like(x)
    if kind == "elu1":
        return np.where(x > 0, 1.0, np.exp(np.minimum(x, 0.0)))
    raise ValueError(kind)


def unit_rows_vjp(x: np.ndarray, g: np.ndarray, length: float = 1.0) -> np.ndarray:
    """The gradient with respect to x of unit_rows(x, length), given the gradient g with
    respect to its result: (length / |x|) (g - u (u . g)) with u = x / |x|, per row; the
    map is constant on a zero row, whose gradient is zero."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    u = np.divide(x, n, out=np.zeros_like(x), where=n > 0)
    f = np.divide(length, n, out=np.zeros_like(n), where=n > 0)
    return f * (g - u * np.sum(u * g, axis=-1, keepdims=True))


def scan_backward(q, k, v, beta, lam, dO, dS=None, *, rule, phi_kind="identity", eps=1e-6,
                  per_channel=False, S0=None, xprev0=None, has0=None, beta_act=None,
                  lam_act=False, qk_norm=None, lam_scaled=False, znorm=False, dz=None):
    """Gradients of L = sum(dO * o) + sum(dS * S_T) (+ sum(dz * z_T) with znorm) with respect
    to every input of scan(),
    for the delta, additive and inner rules with phi identity or elu+1, scalar or
    per-channel lambda (reading D21: the pages give no backward pass).

    Reverse-mode differentiation of the token recurrence, one head at a time: the forward
    steps are rerun keeping each step's state and scalars, then undone from the last
    token to the first, each applying the chain rule to its own formulas
    (S_t = a_t S_{t-1} + eta_t x_t r_t^T with r_t = v_t - S_{t-1}^T x_t, a_t = 1 - eta_t lambda_t,
    eta_t = beta_t / (|x_t|^2 + lambda-hat_t + eps); the additive write gamma_t S_{t-1} +
    beta_t phi(k_t) v_t^T; the read o_t = S_t^T phi(q_t)). lambda-hat's maximum passes its
    gradient to the first channel attaining it.

    With beta_act / lam_act (as in scan(), reading D17) beta and lam hold pre-activations
    z, and their gradients are taken with respect to z: the gate's gradient times the
    activation's derivative (sigmoid: s(1 - s); 2 sigmoid: 2 s(1 - s); softplus: sigmoid(z)).

    With lam_scaled (delta and inner rules, as in scan(), reading D19) the ridge is
    lambda_t |x_t|^2: lambda's gradient is the scaled ridge's times |x_t|^2, and the key
    gains 2 x_t (lambda_t . the scaled ridge's gradient).

    With znorm (additive rule, as in scan(), reading D18) o_t = S_t^T q / (z_t . q + eps):
    the read passes dO_t / den_t to S_t and -(dO_t . o_t) / den_t to den_t, hence q_t z_t
    terms, a gradient G_z of z_t carried back like G (z_t = gamma_t z_{t-1} + beta_t k_t),
    and the initial z (the state's carried-key slot) receives G_z as "xprev0". The final z
    is an output of the scan (the returned state's carried-key slot), so dz [B,H,dk] (None:
    zero), the gradient of L with respect to it, starts G_z; a sequence split over calls
    then chains like one call.

    With qk_norm ("l2" or "rms", identity phi, as in scan()) q, k and the carried key are
    raw and the recurrence sees them rescaled to a fixed length: the gradients with respect
    to the rescaled vectors are taken back through the rescaling (unit_rows_vjp).

    Returns a dict with the gradients "q", "k", "v", "beta", "lam" (None where the input
    is None), "S0" [B,H,dk,dv] and "xprev0" [B,H,dk], in float64.
    """
    if qk_norm is not None:
        if phi_kind != "identity" or qk_norm not in ("l2", "rms"):
            raise ValueError("qk_norm takes the identity feature map and 'l2' or 'rms'")
        length = 1.0 if qk_norm == "l2" else float(np.sqrt(np.asarray(q).shape[-1]))
        # with znorm the carried slot holds z, not a key: it is not rescaled
        key0 = xprev0 is not None and not znorm
        g = scan_backward(unit_rows(q, length), unit_rows(k, length), v, beta, lam, dO, dS,
                          rule=rule, eps=eps, per_channel=per_channel, S0=S0,
                          xprev0=unit_rows(xprev0, length) if key0 else xprev0,
                          has0=has0, beta_act=beta_act, lam_act=lam_act, lam_scaled=lam_scaled,
                          znorm=znorm, dz=dz)
        g["q"] = unit_rows_vjp(q, g["q"], length)
        g["k"] = unit_rows_vjp(k, g["k"], length)
        if key0:
            g["xprev0"] = unit_rows_vjp(xprev0, g["xprev0"], length)
        return g
    q = np.asarray(q, dtype=np.float64)
    B, H, T, dk = q.shape
    dv = np.asarray(v).shape[-1]
    N = B * H
    Q, K, V = _heads(q, 2), _heads(k, 2), _heads(v, 2)
    pv = rule == RULE_DELTA_PV
    Bt = None if beta is None else _heads(beta, 2 if pv else 1)
    Lm = None if lam is None else _heads(lam, 2 if per_channel else 1)
    # gate activations: the activated gates, and each gate's derivative by its
    # pre-activation (1 without an activation)
    dBt = dLm = 1.0
    if Bt is not None and beta_act is not None:
        sb = sigmoid(Bt)
        scale = {"sigmoid": 1.0, "sigmoid2": 2.0}[beta_act]
        Bt, dBt = scale * sb, scale * sb * (1.0 - sb)
    if Lm is not None and lam_act:
        sl = sigmoid(Lm)
        if rule == RULE_ADDITIVE:
            Lm, dLm = sl, sl * (1.0 - sl)
        else:
            Lm, dLm = softplus(Lm), sl
    dOh = _heads(dO, 2)
    dSh = np.zeros((N, dk, dv)) if dS is None else _heads(dS, 2)
    S_init = np.zeros((N, dk, dv)) if S0 is None else _heads(S0, 2)
    x_init = np.zeros((N, dk)) if xprev0 is None else _heads(xprev0, 1)
    h_init = np.zeros(N, dtype=bool) if has0 is None else (np.asarray(has0).reshape(N) != 0)
    shifted = rule in (RULE_DELTA, RULE_INNER, RULE_DELTA_PV)
    if not shifted and rule != RULE_ADDITIVE:
        raise ValueError(rule)
    if pv and per_channel:
        raise ValueError("the per-value-channel rule takes a scalar lambda")
    if lam_scaled and not shifted:
        raise ValueError("lam_scaled takes the delta or inner rule")
    if znorm and rule != RULE_ADDITIVE:
        raise ValueError("znorm takes the additive rule")
    if dz is not None and not znorm:
        raise ValueError("dz is the gradient of the final normaliser (znorm)")
    dzh = np.zeros((N, dk)) if dz is None else _heads(dz, 1)
    if dz is not None and not znorm:
        raise ValueError("dz is the gradient of the final normaliser (znorm)")
    dzh = np.zeros((N, dk)) if dz is None else _heads(dz, 1)

    g = {name: np.zeros_like(a) for name, a in (("q", Q), ("k", K), ("v", V))}
    g["beta"] = None if Bt is None else np.zeros_like(Bt)
    g["lam"] = None if Lm is None else np.zeros_like(Lm)
    g["S0"] = np.zeros((N, dk, dv))
    g["xprev0"] = np.zeros((N, dk))

    for n in range(N):
        # forward, keeping what each step's backward needs
        Sc, xp, hs = S_init[n].copy(), x_init[n].copy(), bool(h_init[n])
        zc = x_init[n].copy()                   # znorm: z lives in the carried-key slot
        steps = []
        for t in range(T):
            qf, kf, vt = phi(Q[n, t], phi_kind), phi(K[n, t], phi_kind), V[n, t]
            Sp = Sc
            if shifted:
                if not hs:
                    steps.append(None)          # no key yet: the step neither decays nor writes
                    Sc = Sp
                else:
                    x = xp
                    if Lm is None:
                        lt, lhat, imax = 0.0, 0.0, None
                    elif per_channel:
                        lt = Lm[n, t]
                        imax = int(np.argmax(lt))
                        lhat = lt[imax]
                    else:
                        lt, lhat, imax = Lm[n, t], Lm[n, t], None
                    # the ridge the step uses: lambda, or lambda |x|^2 (scale-coupled)
                    sc = (x @ x) if lam_scaled else 1.0
                    den = x @ x + lhat * sc + eps
                    eta = Bt[n, t] / den                # per value channel: a d_v-vector
                    a = 1.0 - eta * lt * sc
                    r = vt - Sp.T @ x if rule != RULE_INNER else vt
                    if pv:                              # column j decays by a_j, steps by eta_j
                        Sc = Sp * a[None, :] + np.outer(x, eta * r)
                    else:
                        decay = a[:, None] if per_channel else a
                        Sc = decay * Sp + eta * np.outer(x, r)
                    steps.append((Sp, x, eta, a, den, lt, imax, r, sc))
            else:
                gam = 1.0 if Lm is None else Lm[n, t]
                b = 1.0 if Bt is None else Bt[n, t]
                decay = gam[:, None] if per_channel else gam
                Sc = decay * Sp + b * np.outer(kf, vt)
                zp = zc
                if znorm:
                    zc = gam * zp + b * kf               # gam: a scalar, or per channel
                steps.append((Sp, gam, b, kf, zp, zc))
            steps[-1] = (steps[-1], Sc, qf)
            xp, hs = kf, True

        # backward: G holds dL/dS_t (and Gz dL/dz_t) while step t is undone
        G = dSh[n].copy()
        Gz = dzh[n].copy()
        for t in range(T - 1, -1, -1):
            rec, St, qf = steps[t]
            if znorm:
                zt = rec[5]
                den = zt @ qf + eps
                dnum = dOh[n, t] / den
                dden = -(dOh[n, t] @ (St.T @ qf)) / (den * den)
                g["q"][n, t] += (St @ dnum + zt * dden) * phi_grad(Q[n, t], phi_kind)
                G = G + np.outer(qf, dnum)
                Gz = Gz + qf * dden
            else:
                g["q"][n, t] += (St @ dOh[n, t]) * phi_grad(Q[n, t], phi_kind)
                G = G + np.outer(qf, dOh[n, t])
            if shifted:
                if rec is None:
                    continue                    # S_t = S_{t-1}
                Sp, x, eta, a, den, lt, imax, r, sc = rec
                if pv:
                    # per value channel j: da_j = <G_:j, S_:j>, deta_j = (G^T x)_j r_j - ridge da_j
                    da = np.sum(G * Sp, axis=0)
                    gx = G.T @ x
                    deta = gx * r - lt * sc * da
                    dr = eta * gx
                    dx = G @ (eta * r) - Sp @ dr
                    g["v"][n, t] += dr
                    g["beta"][n, t] += deta / den
                    dden = -np.sum(eta * deta) / den
                    dx = dx + 2.0 * x * dden
                    if Lm is not None:
                        dlt = np.sum(-eta * da) + dden   # the gradient of the ridge used
                        g["lam"][n, t] += dlt * sc
                        if lam_scaled:
                            dx = dx + 2.0 * x * dlt * lt
                    G_prev = G * a[None, :] - np.outer(x, dr)
                else:
                    da = np.sum(G * Sp, axis=1) if per_channel else np.sum(G * Sp)
                    if rule == RULE_DELTA:
                        deta = x @ G @ r
                        dr = eta * (G.T @ x)
                        dx = eta * (G @ r) - Sp @ dr
                        g["v"][n, t] += dr
                        G_prev = (a[:, None] if per_channel else a) * G - np.outer(x, dr)
                    else:
                        deta = x @ G @ V[n, t]
                        dx = eta * (G @ V[n, t])
                        g["v"][n, t] += eta * (G.T @ x)
                        G_prev = (a[:, None] if per_channel else a) * G
                    # a = 1 - eta lambda (lambda: the ridge the step used, lt * sc)
                    deta = deta - (np.sum(lt * sc * da) if per_channel else lt * sc * da)
                    dlt = -eta * da
                    # eta = beta / den, den = |x|^2 + lambda-hat + eps
                    g["beta"][n, t] += deta / den
                    dden = -eta * deta / den
                    dx = dx + 2.0 * x * dden
                    if Lm is not None:
                        if per_channel:
                            dlt = dlt.copy()
                            dlt[imax] += dden
                        else:
                            dlt = dlt + dden
                        # dlt is the gradient of the ridge used; with lam_scaled that ridge is
                        # lt |x|^2
                        g["lam"][n, t] += dlt * sc
                        if lam_scaled:
                            dx = dx + 2.0 * x * (np.sum(dlt * lt) if per_channel else dlt * lt)
                # x_t = phi(k_{t-1}), or the carried key for the sequence's first token
                if t >= 1:
                    g["k"][n, t - 1] += dx * phi_grad(K[n, t - 1], phi_kind)
                else:
                    g["xprev0"][n] += dx
                G = G_prev
            else:
                Sp, gam, b, kf, zp, _ = rec
                if Lm is not None:
                    g["lam"][n, t] += np.sum(G * Sp, axis=1) if per_channel else np.sum(G * Sp)
                    if znorm:
                        g["lam"][n, t] += Gz * zp if per_channel else Gz @ zp
                if Bt is not None:
                    g["beta"][n, t] += kf @ G @ V[n, t] + (Gz @ kf if znorm else 0.0)
                g["k"][n, t] += b * (G @ V[n, t] + Gz) * phi_grad(K[n, t], phi_kind)
                g["v"][n, t] += b * (G.T @ kf)
                G = (gam[:, None] if per_channel else gam) * G
                Gz = gam * Gz
        g["S0"][n] = G
        if znorm:
            g["xprev0"][n] = Gz

    if g["beta"] is not None:
        g["beta"] = g["beta"] * dBt
    if g["lam"] is not None:
        g["lam"] = g["lam"] * dLm
    shapes = {"q": (B, H, T, dk), "k": (B, H, T, dk), "v": (B, H, T, dv),
              "S0": (B, H, dk, dv), "xprev0": (B, H, dk)}
    out = {name: g[name].reshape(shp) for name, shp in shapes.items()}
    out["beta"] = None if g["beta"] is None else g["beta"].reshape(np.asarray(beta).shape)
    out["lam"] = None if g["lam"] is None else g["lam"].reshape(np.asarray(lam).shape)
    return out


def relerr(x, ref) -> float:
    """max|x - ref| / rms(ref), both over the whole tensor, in float64."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    if rms == 0.0:
        return float(np.max(np.abs(x - ref))) if x.size else 0.0
    return float(np.max(np.abs(x - ref)) / rms) if x.size else 0.0
