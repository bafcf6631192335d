"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each pin takes the oracle module as an argument (so the mutation test can run the
same pins on copies of the oracle with a planted mistake) and raises
AssertionError when the oracle disagrees with the pinned fact. None of them
re-types the oracle's recurrence: each compares it with a different statement of
the result (a closed form, a brute-force sum, an invariant, a hand calculation).

Page titles as printed:
  [FWA]  "Fast Weight Attention for Continual Learning" reading notes
  [AFFN] hncyxsy.com blog post "attention is also an FFN"
  [MEM]  "You could have invented transformers from memory" (Alex Wang)
  [FPKM] "Fast-weight Product Key Memory" notes
"""
from __future__ import annotations

from fractions import Fraction as Fr

import numpy as np

DELTA, ADD, INNER = 0, 1, 2


def _unit_rows(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


def _bh(a):
    """Add the (B=1, H=1) leading axes."""
    return np.asarray(a, dtype=np.float64)[None, None]


def pin_p1_outer_product_store(orc):
    """[MEM] outer-product memory store: the additive write with no decay and a
    zero start leaves S = sum_i phi(k_i) v_i^T, the stacked product K^T V (the page's
    W = V^T K, transposed to the d_k x d_v orientation of [AFFN] 4.1)."""
    rng = np.random.default_rng(11)
    for phi_kind in ("identity", "elu1"):
        T, dk, dv = 23, 6, 5
        q = rng.standard_normal((T, dk))
        k = rng.standard_normal((T, dk))
        v = rng.standard_normal((T, dv))
        _, S, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), None, None, rule=ADD, phi_kind=phi_kind)
        if phi_kind == "identity":
            Kf = k
        else:
            Kf = np.where(k > 0, k + 1.0, np.exp(np.minimum(k, 0.0)))
        np.testing.assert_allclose(S[0, 0], Kf.T @ v, rtol=0, atol=1e-12)


def pin_p2_quadratic_form(orc):
    """[AFFN] 2.1: with gamma = 1 the read equals causal linear attention in its
    quadratic form o_t = sum_{j<=t} (phi(q_t) . phi(k_j)) v_j, brute-forced."""
    rng = np.random.default_rng(12)
    T, dk, dv = 13, 5, 4
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    o, _, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), None, None, rule=ADD, phi_kind="elu1")

    def f(x):
        return [xi + 1.0 if xi > 0 else float(np.exp(xi)) for xi in x]

    for t in range(T):
        qt = f(q[t])
        want = [0.0] * dv
        for j in range(t + 1):
            kj = f(k[j])
            w = sum(qt[i] * kj[i] for i in range(dk))
            for c in range(dv):
                want[c] += w * v[j][c]
        np.testing.assert_allclose(o[0, 0, t], want, rtol=0, atol=1e-12)


def pin_p2_decayed_quadratic_form(orc):
    """[AFFN] 3.2, unrolled: with S_t = gamma_t S_{t-1} + phi(k_t) v_t^T,
    o_t = sum_{j<=t} (prod_{j<s<=t} gamma_s) (phi(q_t).phi(k_j)) v_j and
    S_T = sum_j (prod_{s>j} gamma_s) phi(k_j) v_j^T. Scalar and per-channel gamma."""
    rng = np.random.default_rng(13)
    T, dk, dv = 11, 4, 3
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    S0 = rng.standard_normal((dk, dv))
    for per_channel in (False, True):
        gam = rng.uniform(0.3, 1.0, size=(T, dk) if per_channel else (T,))
        beta = rng.uniform(0.5, 1.5, size=T)
        o, S, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(beta), _bh(gam), rule=ADD,
                              phi_kind="identity", per_channel=per_channel, S0=_bh(S0))
        g = gam if per_channel else np.repeat(gam[:, None], dk, axis=1)
        for t in range(T + 1):
            # state after t tokens, channel by channel
            want_S = np.zeros((dk, dv))
            for i in range(dk):
                p0 = 1.0
                for s in range(t):
                    p0 *= g[s, i]
                for c in range(dv):
                    acc = p0 * S0[i, c]
                    for j in range(t):
                        p = 1.0
                        for s in range(j + 1, t):
                            p *= g[s, i]
                        acc += p * beta[j] * k[j, i] * v[j, c]
                    want_S[i, c] = acc
            if t == T:
                np.testing.assert_allclose(S[0, 0], want_S, rtol=0, atol=1e-12)
            if t >= 1:
                np.testing.assert_allclose(o[0, 0, t - 1], want_S.T @ q[t - 1], rtol=0, atol=1e-12)


def pin_p3_first_step_noop(orc):
    """[FWA] 4.1: the first token of a sequence has no causal pair (x_1 = 0,
    eta_1 = 0), so its write leaves S_0 untouched, bit for bit, even with a large
    lambda_1; its read is S_0^T q_1."""
    rng = np.random.default_rng(14)
    dk, dv = 7, 5
    for per_channel in (False, True):
        S0 = rng.standard_normal((2, 3, dk, dv))
        q = rng.standard_normal((2, 3, 1, dk))
        k = rng.standard_normal((2, 3, 1, dk))
        v = rng.standard_normal((2, 3, 1, dv))
        beta = rng.uniform(0.1, 1.9, size=(2, 3, 1))
        lam = rng.uniform(0.5, 5.0, size=(2, 3, 1, dk) if per_channel else (2, 3, 1))
        o, S, xp, has = orc.scan(q, k, v, beta, lam, rule=DELTA, per_channel=per_channel, S0=S0)
        assert np.array_equal(S, S0), "step 1 must not change S"
        np.testing.assert_allclose(o[:, :, 0], np.einsum("bhij,bhi->bhj", S0, q[:, :, 0]),
                                   rtol=0, atol=1e-12)
        assert np.array_equal(xp, k[:, :, 0]) and np.all(has == 1)


def pin_p4_nlms_rewrite(orc):
    """[FWA] 4.2: with lambda = eps = 0 the rule is NLMS; with beta = 1 the step
    rewrites the memory so that it recalls the newest target exactly
    (S_t^T x_t = y_t, the one-step rewrite of [FPKM] 3.2.1). Read with q_t = k_{t-1}."""
    rng = np.random.default_rng(15)
    T, dk, dv = 40, 6, 4
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    q = np.concatenate([rng.standard_normal((1, dk)), k[:-1]], axis=0)
    S0 = rng.standard_normal((dk, dv))
    o, _, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(np.ones(T)), _bh(np.zeros(T)),
                          rule=DELTA, eps=0.0, S0=_bh(S0))
    np.testing.assert_allclose(o[0, 0, 1:], v[1:], rtol=0, atol=1e-10)


def pin_p5_orthonormal_recall(orc):
    """[MEM] recall with orthonormal keys has no interference, so recall is exact.
    Delta rule, beta = 1, lambda = eps = 0, S_0 = 0, shifted pairing: the memory
    maps k_j to v_{j+1} for every written key."""
    rng = np.random.default_rng(16)
    dk, dv = 8, 5
    T = dk + 1
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = np.concatenate([Qm.T, rng.standard_normal((1, dk))], axis=0)   # k_0..k_{T-2} orthonormal
    v = rng.standard_normal((T, dv))
    q = rng.standard_normal((T, dk))
    _, S, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(np.ones(T)), None, rule=DELTA, eps=0.0)
    for j in range(T - 1):
        np.testing.assert_allclose(S[0, 0].T @ k[j], v[j + 1], rtol=0, atol=1e-12)


def _ridge_loss(S, x, y, lam_vec):
    r = S.T @ x - y
    return 0.5 * float(r @ r) + 0.5 * float(np.sum(lam_vec[:, None] * S * S))


def pin_p6_descent_lemma(orc, trials=400):
    """[FWA] 3.2 and 4.2 (Lemma 3.1): each step does not increase the instantaneous
    ridge loss l_t(S) = 1/2 ||S^T x_t - y_t||^2 + 1/2 sum_i lambda_{t,i} ||S_{i,:}||^2
    for beta in (0, 2). Per-channel lambda uses the max-channel denominator
    (reading D1), which bounds the loss's curvature; trials include large lambda and
    small keys so that a weaker denominator would fail."""
    rng = np.random.default_rng(17)
    for trial in range(trials):
        per_channel = trial % 2 == 1
        dk, dv = 5, 3
        S = rng.standard_normal((dk, dv)) * rng.uniform(0.1, 3.0)
        xp = rng.standard_normal(dk) * rng.uniform(0.05, 2.0)
        for _ in range(3):
            k = rng.standard_normal(dk) * rng.uniform(0.05, 2.0)
            v = rng.standard_normal(dv) * rng.uniform(0.1, 3.0)
            beta = rng.uniform(0.01, 1.99)
            lam = rng.uniform(0.0, 4.0, size=dk) if per_channel else rng.uniform(0.0, 4.0)
            lam_arr = lam[None, None, :] if per_channel else np.array([[lam]])
            _, S_new, xp_new, _ = orc.step(
                rng.standard_normal((1, 1, dk)), k[None, None], v[None, None],
                np.array([[beta]]), lam_arr, rule=DELTA, eps=1e-6, per_channel=per_channel,
                S0=S[None, None], xprev0=xp[None, None], has0=np.array([[1]]))
            lam_vec = lam if per_channel else np.full(dk, lam)
            before = _ridge_loss(S, xp, v, lam_vec)
            after = _ridge_loss(S_new[0, 0], xp, v, lam_vec)
            assert after <= before * (1 + 1e-12) + 1e-14, (trial, before, after)
            S, xp = S_new[0, 0], xp_new[0, 0]


def pin_p7_zero_beta(orc):
    """[FWA] 3.2: beta = 0 makes eta = 0: no decay and no write, so S_t = S_0 and
    o_t = S_0^T q_t at every step."""
    rng = np.random.default_rng(18)
    T, dk, dv = 9, 6, 4
    S0 = rng.standard_normal((dk, dv))
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    lam = rng.uniform(0.1, 2.0, size=T)
    o, S, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(np.zeros(T)), _bh(lam), rule=DELTA,
                          S0=_bh(S0))
    assert np.array_equal(S[0, 0], S0)
    np.testing.assert_allclose(o[0, 0], q @ S0, rtol=0, atol=1e-12)


def pin_p8_per_channel_equal(orc):
    """Reading D1 reduces to the scalar rule when every channel has the same lambda."""
    rng = np.random.default_rng(19)
    T, dk, dv = 17, 6, 5
    q = rng.standard_normal((2, 2, T, dk))
    k = rng.standard_normal((2, 2, T, dk))
    v = rng.standard_normal((2, 2, T, dv))
    beta = rng.uniform(0.1, 1.9, size=(2, 2, T))
    lam = rng.uniform(0.0, 0.5, size=(2, 2, T))
    a = orc.scan(q, k, v, beta, lam, rule=DELTA)
    b = orc.scan(q, k, v, beta, np.repeat(lam[..., None], dk, axis=-1), rule=DELTA,
                 per_channel=True)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-13)


def pin_p9_hand_delta(orc):
    """[AFFN] 5.2 advises checking a length-2, d = 4 case by hand. Delta rule,
    phi = id, eps = 0, S_0 = 0; token 1 has no pair. Worked by hand:
      t=2: x = k_1 = e_1, eta = 1/(1+1) = 1/2, r = v_2, S_2 = 1/2 e_1 v_2^T
           -> row 0 = (1/2, 1, 3/2, 2)
      t=3: x = k_2 = (1,1,0,0), ||x||^2 = 2, eta = 1/(2+1) = 1/3,
           S_2^T x = (1/2, 1, 3/2, 2), r = (7/2, 2, 1/2, -1), decay 2/3
           row 0 = 2/3 (1/2,1,3/2,2) + 1/3 r = (3/2, 4/3, 7/6, 1)
           row 1 = 1/3 r = (7/6, 2/3, 1/6, -1/3)
      reads: o_1 = 0, o_2 = S_2^T (1,0,0,1) = row 0 of S_2,
             o_3 = S_3^T (0,1,1,0) = row 1 of S_3."""
    k = np.array([[1, 0, 0, 0], [1, 1, 0, 0], [0, 0, 1, 0]], dtype=np.float64)
    v = np.array([[9, 9, 9, 9], [1, 2, 3, 4], [4, 3, 2, 1]], dtype=np.float64)
    q = np.array([[1, 1, 1, 1], [1, 0, 0, 1], [0, 1, 1, 0]], dtype=np.float64)
    beta = np.array([1.0, 1.0, 1.0])
    lam = np.array([5.0, 1.0, 1.0])          # lambda_1 is irrelevant: step 1 is a no-op
    o, S, xp, has = orc.scan(_bh(q), _bh(k), _bh(v), _bh(beta), _bh(lam), rule=DELTA, eps=0.0)
    S3 = [[Fr(3, 2), Fr(4, 3), Fr(7, 6), Fr(1)],
          [Fr(7, 6), Fr(2, 3), Fr(1, 6), Fr(-1, 3)],
          [0, 0, 0, 0], [0, 0, 0, 0]]
    o_want = [[0, 0, 0, 0],
              [Fr(1, 2), Fr(1), Fr(3, 2), Fr(2)],
              [Fr(7, 6), Fr(2, 3), Fr(1, 6), Fr(-1, 3)]]
    np.testing.assert_allclose(S[0, 0], np.array(S3, dtype=np.float64), rtol=0, atol=1e-14)
    np.testing.assert_allclose(o[0, 0], np.array(o_want, dtype=np.float64), rtol=0, atol=1e-14)
    assert np.array_equal(xp[0, 0], k[2]) and has[0, 0] == 1


def pin_p9_hand_additive(orc):
    """Additive rule with phi = elu+1 ([AFFN] 4.1) and gamma = 1/2, worked by hand:
      phi(k_1) = phi(0,1) = (1,2), phi(k_2) = phi(1,0) = (2,1), v_1 = (1,0), v_2 = (0,1)
      S_1 = phi(k_1) v_1^T = [[1,0],[2,0]]
      S_2 = 1/2 S_1 + phi(k_2) v_2^T = [[1/2,2],[1,1]]
      o_1 = S_1^T phi(0,0) = S_1^T (1,1) = (3,0)
      o_2 = S_2^T phi(1,1) = S_2^T (2,2) = (3,6)"""
    k = np.array([[0.0, 1.0], [1.0, 0.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0]])
    q = np.array([[0.0, 0.0], [1.0, 1.0]])
    gam = np.array([0.5, 0.5])
    o, S, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), None, _bh(gam), rule=ADD, phi_kind="elu1")
    np.testing.assert_allclose(S[0, 0], [[0.5, 2.0], [1.0, 1.0]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0, 0], [[3.0, 0.0], [3.0, 6.0]], rtol=0, atol=1e-15)


def pin_p10_state_carry(orc):
    """Reading D3: a scan split in two with the state (S, xprev, has_prev) carried,
    and T single-token steps, both equal one scan over the whole sequence."""
    rng = np.random.default_rng(20)
    B, H, T, dk, dv = 2, 2, 12, 5, 4
    for rule in (DELTA, ADD):
        q = rng.standard_normal((B, H, T, dk))
        k = rng.standard_normal((B, H, T, dk))
        v = rng.standard_normal((B, H, T, dv))
        beta = rng.uniform(0.1, 1.9, size=(B, H, T))
        lam = rng.uniform(0.0, 0.9, size=(B, H, T)) if rule == DELTA else rng.uniform(0.5, 1.0, size=(B, H, T))
        phi_kind = "identity" if rule == DELTA else "elu1"
        full = orc.scan(q, k, v, beta, lam, rule=rule, phi_kind=phi_kind)
        T1 = 5
        a = orc.scan(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], beta[:, :, :T1], lam[:, :, :T1],
                     rule=rule, phi_kind=phi_kind)
        b = orc.scan(q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], beta[:, :, T1:], lam[:, :, T1:],
                     rule=rule, phi_kind=phi_kind, S0=a[1], xprev0=a[2], has0=a[3])
        np.testing.assert_allclose(np.concatenate([a[0], b[0]], axis=2), full[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(b[1], full[1], rtol=0, atol=1e-12)
        S, xp, has = None, None, None
        outs = []
        for t in range(T):
            o, S, xp, has = orc.step(q[:, :, t], k[:, :, t], v[:, :, t], beta[:, :, t],
                                     lam[:, :, t], rule=rule, phi_kind=phi_kind,
                                     S0=S, xprev0=xp, has0=has)
            outs.append(o)
        np.testing.assert_allclose(np.stack(outs, axis=2), full[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(S, full[1], rtol=0, atol=1e-12)


def pin_p11_interference_ratio(orc):
    """[MEM] recall produces interference: storing M random unit keys additively in
    d_k dimensions and recalling with a stored key gives
    E ||interference||^2 / ||signal||^2 = (M - 1)/d_k. Checked statistically (+-10%)."""
    rng = np.random.default_rng(21)
    dk, dv = 64, 64
    for M in (16, 64, 128):
        ratios = []
        for _ in range(6):
            keys = _unit_rows(rng, M, dk)
            vals = _unit_rows(rng, M, dv)
            # M writes, then M read-only tokens (k = 0, v = 0) that query each stored key
            k = np.concatenate([keys, np.zeros((M, dk))])
            v = np.concatenate([vals, np.zeros((M, dv))])
            q = np.concatenate([np.zeros((M, dk)), keys])
            o, _, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), None, None, rule=ADD)
            rec = o[0, 0, M:]
            ratios.extend(np.sum((rec - vals) ** 2, axis=1) / np.sum(vals ** 2, axis=1))
        want = (M - 1) / dk
        got = float(np.mean(ratios))
        assert abs(got - want) <= 0.1 * want, (M, got, want)


def pin_p12_min_norm_store(orc):
    """[MEM] optimal linear memory store: for M <= d_k independent keys the
    least-squares store of minimum norm recalls exactly, W = V^T (K K^T)^{-1} K.
    Sweeping the M pairs repeatedly through the NLMS limit of the delta rule from
    S_0 = 0 (Kaczmarz's projections) converges to it; in the d_k x d_v orientation
    S* = K^T (K K^T)^{-1} V."""
    rng = np.random.default_rng(22)
    M, dk, dv = 5, 8, 3
    keys = rng.standard_normal((M, dk))
    vals = rng.standard_normal((M, dv))
    sweeps = 300
    T = M * sweeps + 1
    idx_k = np.arange(T) % M
    idx_v = (np.arange(T) - 1) % M          # token t carries v = vals[(t-1) mod M]: pair (k_{t-1}, v_t)
    k = keys[idx_k]
    v = vals[idx_v]
    q = np.zeros((T, dk))
    _, S, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(np.ones(T)), None, rule=DELTA, eps=0.0)
    S_star = keys.T @ np.linalg.solve(keys @ keys.T, vals)
    np.testing.assert_allclose(S[0, 0], S_star, rtol=0, atol=1e-9)


def _shifted_eta(k, beta, lam, eps):
    """eta_t of the shifted pair for one head, brute force: x_1 = 0 with eta_1 = 0,
    then x_t = k_{t-1}, eta_t = beta_t / (|x_t|^2 + lambda_t + eps) ([FWA] 4.1, 4.2)."""
    T = k.shape[0]
    eta = np.zeros(T)
    for t in range(1, T):
        eta[t] = beta[t] / (float(k[t - 1] @ k[t - 1]) + lam[t] + eps)
    return eta


def pin_p13_inner_hebbian_sum(orc):
    """[FWA] 4.3: with lambda = 0 the inner-product rule is a pure additive write of
    the shifted pair, so S_T = sum_{t>=2} eta_t k_{t-1} v_t^T and
    o_t = sum_{2<=j<=t} eta_j (q_t . k_{j-1}) v_j, both brute-forced."""
    rng = np.random.default_rng(31)
    T, dk, dv, eps = 12, 5, 3, 1e-3
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0.1, 1.9, T)
    o, S, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(beta), None, rule=INNER, eps=eps)
    eta = _shifted_eta(k, beta, np.zeros(T), eps)
    S_ref = np.zeros((dk, dv))
    for j in range(1, T):
        S_ref += eta[j] * np.outer(k[j - 1], v[j])
    np.testing.assert_allclose(S[0, 0], S_ref, rtol=0, atol=1e-12)
    for t in range(T):
        ref = np.zeros(dv)
        for j in range(1, t + 1):
            ref += eta[j] * float(q[t] @ k[j - 1]) * v[j]
        np.testing.assert_allclose(o[0, 0, t], ref, rtol=0, atol=1e-12)


def pin_p14_inner_decayed_sum(orc):
    """[FWA] 4.3 with lambda > 0, unrolled: each write eta_j x_j v_j^T is scaled by the
    decays of the later steps, S_T = sum_j diag(prod_{s>j} a_s) eta_j x_j v_j^T with
    a_s = 1 - eta_s lambda_s (a d_k-vector for per-channel lambda, eta's denominator
    taking the channel max, reading D1), starting from a nonzero S_0 that decays as a
    whole. The read o_t = S_t^T q_t is checked against the same unrolled sum."""
    rng = np.random.default_rng(32)
    T, dk, dv, eps = 10, 4, 3, 1e-6
    for per_channel in (False, True):
        q = rng.standard_normal((T, dk))
        k = rng.standard_normal((T, dk))
        v = rng.standard_normal((T, dv))
        beta = rng.uniform(0.1, 1.9, T)
        lam = rng.uniform(0.05, 0.6, (T, dk) if per_channel else T)
        S0 = rng.standard_normal((dk, dv))
        o, S, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(beta), _bh(lam), rule=INNER, eps=eps,
                              per_channel=per_channel, S0=_bh(S0))
        lam_hat = lam.max(axis=1) if per_channel else lam
        eta = _shifted_eta(k, beta, lam_hat, eps)
        a = [1.0 - eta[s] * (lam[s] if per_channel else np.full(dk, lam[s])) for s in range(T)]

        def state_at(t):  # S_t for t = 0..T-1 (after step t), brute force
            acc = S0 * np.prod([a[s] for s in range(0, t + 1)], axis=0)[:, None]
            for j in range(1, t + 1):
                dec = np.prod([a[s] for s in range(j + 1, t + 1)], axis=0) if j < t else np.ones(dk)
                acc = acc + (dec * eta[j] * k[j - 1])[:, None] * v[j][None, :]
            return acc

        np.testing.assert_allclose(S[0, 0], state_at(T - 1), rtol=0, atol=1e-12)
        for t in range(T):
            np.testing.assert_allclose(o[0, 0, t], state_at(t).T @ q[t], rtol=0, atol=1e-12)


def _inner_loss(S, x, y, lam):
    return -float(x @ S @ y) + 0.5 * lam * float(np.sum(S * S))


def pin_p15_inner_gradient_step(orc, trials=300):
    """[FWA] 4.3: each step is a gradient step of size eta_t on the instantaneous loss
    l_t(S) = -<S^T x_t, y_t> + (lambda_t/2)|S|_F^2. That loss is quadratic with
    Hessian lambda_t I, so the step changes it by exactly
    -eta |g|^2 (1 - lambda eta / 2) with g = lambda S_{t-1} - x_t y_t^T, which is a
    decrease whenever beta_t in (0, 2)."""
    rng = np.random.default_rng(33)
    dk, dv = 5, 4
    for _ in range(trials):
        S0 = rng.standard_normal((dk, dv))
        x = rng.standard_normal(dk) * rng.uniform(0.1, 3.0)
        y = rng.standard_normal(dv)
        beta = rng.uniform(0.05, 1.95)
        lam = rng.uniform(0.01, 2.0)
        eps = 1e-6
        k = np.stack([x, rng.standard_normal(dk)])
        v = np.stack([rng.standard_normal(dv), y])
        _, S, _, _ = orc.scan(_bh(np.zeros((2, dk))), _bh(k), _bh(v), _bh(np.array([1.0, beta])),
                              _bh(np.array([0.3, lam])), rule=INNER, eps=eps, S0=_bh(S0))
        # step 1 has no previous key, so S after step 1 is S0 and step 2 writes (x, y)
        eta = beta / (float(x @ x) + lam + eps)
        g = lam * S0 - np.outer(x, y)
        before, after = _inner_loss(S0, x, y, lam), _inner_loss(S[0, 0], x, y, lam)
        expect = -eta * float(np.sum(g * g)) * (1.0 - 0.5 * lam * eta)
        assert after <= before + 1e-12
        assert abs((after - before) - expect) <= 1e-10 * max(1.0, abs(expect))


def pin_p16_inner_first_step_noop(orc):
    """[FWA] 4.1: x_1 = 0 and eta_1 = 0 make the first write of a sequence a no-op for
    the inner-product rule too: S_1 equals S_0 exactly and o_1 = S_0^T q_1."""
    rng = np.random.default_rng(34)
    dk, dv = 6, 5
    S0 = rng.standard_normal((dk, dv))
    q = rng.standard_normal((1, dk))
    k = rng.standard_normal((1, dk))
    v = rng.standard_normal((1, dv))
    o, S, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(np.array([1.7])), _bh(np.array([0.9])),
                          rule=INNER, S0=_bh(S0))
    assert np.array_equal(S[0, 0], S0)
    np.testing.assert_allclose(o[0, 0, 0], S0.T @ q[0], rtol=0, atol=1e-13)


def pin_p17_inner_is_shifted_linear_attention(orc):
    """[FWA] 4.3 calls the inner-product rule the shifted-pair version of linear
    attention's accumulation: it equals the additive rule (pinned by P1, P2, P2')
    run on the keys shifted by one token, with write scale eta_t and retention
    1 - eta_t lambda_t computed here by brute force."""
    rng = np.random.default_rng(35)
    T, dk, dv, eps = 15, 6, 4, 1e-6
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0.1, 1.9, T)
    lam = rng.uniform(0.0, 0.5, T)
    o, S, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(beta), _bh(lam), rule=INNER, eps=eps)
    eta = _shifted_eta(k, beta, lam, eps)
    k_shift = np.vstack([np.zeros((1, dk)), k[:-1]])
    o2, S2, _, _ = orc.scan(_bh(q), _bh(k_shift), _bh(v), _bh(eta), _bh(1.0 - eta * lam), rule=ADD)
    np.testing.assert_allclose(S[0, 0], S2[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o[0, 0], o2[0, 0], rtol=0, atol=1e-12)


def pin_p9_hand_inner(orc):
    """A case worked by hand ([AFFN] 5.2's advice to check a tiny case), in exact
    fractions. d_k = 2, d_v = 1, beta = 1, lambda = 1/2, eps = 0, q_t = (1, 1),
    k_1 = (1, 0), k_2 = (0, 2), v = (5, 3, 7):
      t = 1: no previous key, S_1 = 0, o_1 = 0;
      t = 2: x = (1, 0), eta = 1/(1 + 1/2) = 2/3, a = 2/3, S_2 = (2/3)(1, 0)^T 3 = (2, 0)^T,
             o_2 = 2;
      t = 3: x = (0, 2), eta = 1/(4 + 1/2) = 2/9, a = 8/9,
             S_3 = (8/9)(2, 0)^T + (2/9)(0, 2)^T 7 = (16/9, 28/9)^T, o_3 = 44/9."""
    q = np.ones((3, 2))
    k = np.array([[1.0, 0.0], [0.0, 2.0], [3.0, -1.0]])
    v = np.array([[5.0], [3.0], [7.0]])
    o, S, xp, h = orc.scan(_bh(q), _bh(k), _bh(v), _bh(np.ones(3)), _bh(np.full(3, 0.5)),
                           rule=INNER, eps=0.0)
    exp_o = [Fr(0), Fr(2), Fr(44, 9)]
    exp_S = [Fr(16, 9), Fr(28, 9)]
    for t in range(3):
        assert abs(o[0, 0, t, 0] - float(exp_o[t])) < 1e-14
    for i in range(2):
        assert abs(S[0, 0, i, 0] - float(exp_S[i])) < 1e-14
    assert np.array_equal(xp[0, 0], k[2]) and h[0, 0] == 1


def _qk_cases(rng, T, dk, dv):
    """Raw (unnormalised) inputs with a spread of token norms, and gates for each rule."""
    q = rng.standard_normal((T, dk)) * rng.uniform(0.2, 5.0, (T, 1))
    k = rng.standard_normal((T, dk)) * rng.uniform(0.2, 5.0, (T, 1))
    v = rng.standard_normal((T, dv))
    beta = rng.uniform(0.1, 1.9, T)
    lam = {DELTA: rng.uniform(0.0, 0.3, T), INNER: rng.uniform(0.0, 0.3, T),
           ADD: rng.uniform(0.7, 1.0, T)}
    return q, k, v, beta, lam


def pin_p18_qk_norm_is_the_rule_on_normalised_inputs(orc):
    """[FWA] 4.5 normalises the query and key projections: with qk_norm the scan equals
    the plain scan on q and k rescaled here, by an independent route, to RMS 1
    (RMSNorm with unit gain: divide by sqrt(mean of squares)) or to unit length.
    The state's carried key is the raw last key (reading D16)."""
    rng = np.random.default_rng(36)
    T, dk, dv = 14, 6, 4
    for rule in (DELTA, INNER, ADD):
        q, k, v, beta, lam = _qk_cases(rng, T, dk, dv)
        for mode in ("l2", "rms"):
            rms_q = np.sqrt(np.mean(q * q, axis=1, keepdims=True))
            rms_k = np.sqrt(np.mean(k * k, axis=1, keepdims=True))
            scale = 1.0 if mode == "rms" else 1.0 / np.sqrt(dk)
            qn, kn = q / rms_q * scale, k / rms_k * scale
            b = beta if rule != ADD else None
            o, S, xp, h = orc.scan(_bh(q), _bh(k), _bh(v), None if b is None else _bh(b), _bh(lam[rule]),
                                   rule=rule, eps=1e-6, qk_norm=mode)
            o2, S2, _, _ = orc.scan(_bh(qn), _bh(kn), _bh(v), None if b is None else _bh(b),
                                    _bh(lam[rule]), rule=rule, eps=1e-6)
            np.testing.assert_allclose(o[0, 0], o2[0, 0], rtol=0, atol=1e-11)
            np.testing.assert_allclose(S[0, 0], S2[0, 0], rtol=0, atol=1e-11)
            assert np.array_equal(xp[0, 0], k[-1]) and h[0, 0] == 1
    # a zero query or key stays zero: with every key zero, nothing is written
    q, k, v, beta, lam = _qk_cases(rng, T, dk, dv)
    o, S, _, _ = orc.scan(_bh(q), _bh(np.zeros_like(k)), _bh(v), _bh(beta), _bh(lam[DELTA]), rule=DELTA,
                          qk_norm="l2")
    assert np.all(S == 0.0) and np.all(o == 0.0)


def pin_p19_qk_norm_scale_invariance(orc):
    """A consequence of normalising q and k: multiplying each token's q and k by any
    positive number changes nothing but the carried raw key, for every rule and across
    a call boundary that carries the key."""
    rng = np.random.default_rng(37)
    T, dk, dv, T1 = 16, 5, 3, 7
    for rule in (DELTA, INNER, ADD):
        q, k, v, beta, lam = _qk_cases(rng, T, dk, dv)
        cq, ck = rng.uniform(0.01, 100.0, (T, 1)), rng.uniform(0.01, 100.0, (T, 1))
        b = beta if rule != ADD else None

        def run(qq, kk):
            sl = lambda a, s_: None if a is None else _bh(a[s_])
            first, second = slice(0, T1), slice(T1, None)
            o1, S1, x1, h1 = orc.scan(sl(qq, first), sl(kk, first), sl(v, first), sl(b, first),
                                      sl(lam[rule], first), rule=rule, qk_norm="rms")
            o2, S2, x2, h2 = orc.scan(sl(qq, second), sl(kk, second), sl(v, second), sl(b, second),
                                      sl(lam[rule], second), rule=rule, qk_norm="rms", S0=S1,
                                      xprev0=x1, has0=h1)
            return np.concatenate([o1[0, 0], o2[0, 0]]), S2[0, 0], x2[0, 0]

        o, S, xp = run(q, k)
        oc, Sc, xpc = run(q * cq, k * ck)
        np.testing.assert_allclose(oc, o, rtol=0, atol=1e-10 * max(1.0, np.abs(o).max()))
        np.testing.assert_allclose(Sc, S, rtol=0, atol=1e-10 * max(1.0, np.abs(S).max()))
        np.testing.assert_allclose(xpc, k[-1] * ck[-1], rtol=1e-15, atol=0)


def pin_p20_gate_preactivations(orc):
    """Gates passed as pre-activations z ([FWA] 4.2 keeps beta in (0, 2); the ridge is
    nonnegative and the additive retention lies in (0, 1)): the scan equals the plain
    scan on gates activated here by independent formulas, sigmoid(z) = (1 + tanh(z/2))/2
    and softplus(z) = logaddexp(0, z); and the special values sigmoid(0) = 1/2,
    softplus(0) = ln 2 hold."""
    rng = np.random.default_rng(38)
    T, dk, dv = 12, 5, 4
    sig = lambda z: 0.5 * (1.0 + np.tanh(0.5 * z))
    sp = lambda z: np.logaddexp(0.0, z)
    assert orc.sigmoid(np.array(0.0)) == 0.5 and abs(orc.softplus(np.array(0.0)) - np.log(2.0)) < 1e-16
    for rule in (DELTA, INNER, ADD):
        for per_channel in (False, True):
            q, k, v = (rng.standard_normal((T, d)) for d in (dk, dk, dv))
            zb = rng.standard_normal(T) * 2
            zl = rng.standard_normal((T, dk) if per_channel else T) * 2 - 2
            for act, scale in (("sigmoid", 1.0), ("sigmoid2", 2.0)):
                lam_ref = sig(zl) if rule == ADD else sp(zl)
                o, S, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(zb), _bh(zl), rule=rule,
                                      per_channel=per_channel, beta_act=act, lam_act=True)
                o2, S2, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(scale * sig(zb)), _bh(lam_ref),
                                        rule=rule, per_channel=per_channel)
                np.testing.assert_allclose(o[0, 0], o2[0, 0], rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(S[0, 0], S2[0, 0], rtol=1e-12, atol=1e-12)


def pin_p21_normalised_linear_attention(orc):
    """[AFFN] 4.2: with the normaliser, the read is the quadratic form divided by its
    weights, o_t = sum_{j<=t} w_tj v_j / (sum_{j<=t} w_tj + eps) with
    w_tj = (prod_{s=j+1..t} gamma_s) beta_j (phi(q_t) . phi(k_j)), brute-forced; and with
    eps = 0 every value equal to one vector c makes every read exactly c (a weighted
    average of equal values)."""
    rng = np.random.default_rng(39)
    T, dk, dv, eps = 11, 5, 4, 1e-3
    for per_channel in (False, True):
        q = rng.standard_normal((T, dk))
        k = rng.standard_normal((T, dk))
        v = rng.standard_normal((T, dv))
        beta = rng.uniform(0.2, 1.5, T)
        gam = rng.uniform(0.6, 1.0, (T, dk) if per_channel else T)
        o, _, z, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(beta), _bh(gam), rule=ADD, phi_kind="elu1",
                              per_channel=per_channel, eps=eps, znorm=True)
        fq = np.where(q > 0, q + 1.0, np.exp(np.minimum(q, 0.0)))
        fk = np.where(k > 0, k + 1.0, np.exp(np.minimum(k, 0.0)))
        g = gam if per_channel else np.repeat(gam[:, None], dk, axis=1)
        z_ref = np.zeros(dk)
        for t in range(T):
            num, den = np.zeros(dv), 0.0
            for j in range(t + 1):
                dec = np.prod(g[j + 1:t + 1], axis=0) if j < t else np.ones(dk)
                w = beta[j] * float(np.sum(fq[t] * dec * fk[j]))
                num += w * v[j]
                den += w
            np.testing.assert_allclose(o[0, 0, t], num / (den + eps), rtol=1e-11, atol=1e-12)
            z_ref = g[t] * z_ref + beta[t] * fk[t]
        np.testing.assert_allclose(z[0, 0], z_ref, rtol=1e-12)
    c = rng.standard_normal(dv)
    o, _, _, _ = orc.scan(_bh(q), _bh(k), _bh(np.tile(c, (T, 1))), _bh(beta), _bh(gam[:, 0] if gam.ndim == 2 else gam),
                          rule=ADD, phi_kind="elu1", eps=0.0, znorm=True)
    np.testing.assert_allclose(o[0, 0], np.tile(c, (T, 1)), rtol=1e-12, atol=1e-12)


def pin_relerr_metric(orc):
    """The parity metric max|x - ref| / rms(ref) on a case worked by hand."""
    ref = np.array([3.0, -4.0])          # rms = sqrt((9 + 16)/2) = 5/sqrt(2)
    x = np.array([3.5, -4.0])
    assert abs(orc.relerr(x, ref) - 0.5 / (5.0 / np.sqrt(2.0))) < 1e-15


def pin_p22_scale_coupled_ridge(orc):
    """[FWA] 4.5: with the ridge coupled to the energy of the written key, the decay
    does not depend on the input scale. With eps = 0, multiplying every q and k by s > 0
    (and S0 by 1/s) leaves every read unchanged and divides the state by s: eta scales by
    1/s^2, eta x by 1/s, eta lambda not at all. Checked for the delta and inner rules, with
    scalar and per-channel base ridges; the plain ridge lacks the property (checked too).
    Hand case, one write: x = (3, 4), base ridge 0.2, beta = 1, eps = 0, S0 = (1, 2)^T,
    v = 10. Then lambda = 0.2 * 25 = 5, eta = 1/30, decay 5/6, and the residual is
    10 - 11 = -1, so the delta rule gives S = (11/15, 23/15); the inner rule writes v
    itself and gives S = (11/6, 3)."""
    rng = np.random.default_rng(40)
    T, dk, dv, s = 14, 5, 3, 7.3
    for rule in (DELTA, INNER):
        for per_channel in (False, True):
            q, k, v = (rng.standard_normal((T, d)) for d in (dk, dk, dv))
            beta = rng.uniform(0.2, 1.8, T)
            lam = rng.uniform(0.05, 0.5, (T, dk) if per_channel else T)
            S0 = rng.standard_normal((1, 1, dk, dv))

            def run(c, scaled):
                return orc.scan(_bh(c * q), _bh(c * k), _bh(v), _bh(beta), _bh(lam), rule=rule,
                                per_channel=per_channel, eps=0.0, S0=S0 / c, lam_scaled=scaled)

            o, S, _, _ = run(1.0, True)
            o2, S2, _, _ = run(s, True)
            np.testing.assert_allclose(o2, o, rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(S2 * s, S, rtol=1e-10, atol=1e-12)
            o3 = run(1.0, False)[0]
            o4 = run(s, False)[0]
            assert np.max(np.abs(o4 - o3)) > 1e-3
    q = np.array([[0.0, 1.0], [1.0, 0.0]])
    k = np.array([[3.0, 4.0], [1.0, 1.0]])
    v = np.array([[5.0], [10.0]])
    S0 = np.array([[1.0], [2.0]])[None, None]
    for rule, S_hand in ((DELTA, [11 / 15, 23 / 15]), (INNER, [11 / 6, 3.0])):
        o, S, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(np.ones(2)), _bh(np.array([0.7, 0.2])),
                              rule=rule, eps=0.0, S0=S0, lam_scaled=True)
        np.testing.assert_allclose(S[0, 0, :, 0], S_hand, rtol=1e-14)
        np.testing.assert_allclose(o[0, 0, :, 0], [2.0, S_hand[0]], rtol=1e-14)


def pin_p23_per_value_channel_rule(orc):
    """[FWA] 4.4 (Falcon-2). Four checks.
    (a) Equal step sizes on every value channel give the delta rule.
    (b) The objective separates over the value channels, so column j of the state and
        of the reads equals a one-column delta rule with that channel's beta (d_k != d_v,
        so an axis slip cannot hide).
    (c) The per-step descent lemma holds for every channel's own loss
        l_j(S) = (v_j - S[:, j] . x)^2 / 2 + lambda |S[:, j]|^2 / 2, for beta_j in (0, 2).
    (d) Hand case, one write. S0 = [[1, 2], [3, 4]], x = (3, 4), v = (10, 20),
        beta = (1, 1/2), lambda = 5, eps = 0. Then eta = (1/30, 1/60), the decays are
        (5/6, 11/12) and r = v - S0^T x = (-5, -2), so S = [[1/3, 26/15], [11/6, 53/15]]."""
    rng = np.random.default_rng(41)
    T, dk, dv = 13, 5, 3
    PV = orc.RULE_DELTA_PV
    for scaled in (False, True):
        q, k = rng.standard_normal((T, dk)), rng.standard_normal((T, dk))
        v = rng.standard_normal((T, dv))
        lam = rng.uniform(0.01, 0.5, T)
        S0 = rng.standard_normal((1, 1, dk, dv))
        b1 = rng.uniform(0.1, 1.9, T)
        o, S, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(np.repeat(b1[:, None], dv, 1)), _bh(lam),
                              rule=PV, S0=S0, lam_scaled=scaled)
        o_d, S_d, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(b1), _bh(lam), rule=DELTA, S0=S0,
                                  lam_scaled=scaled)
        np.testing.assert_allclose(o, o_d, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(S, S_d, rtol=1e-12, atol=1e-13)
        bpv = rng.uniform(0.1, 1.9, (T, dv))
        o, S, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(bpv), _bh(lam), rule=PV, S0=S0,
                              lam_scaled=scaled)
        for j in range(dv):
            o_j, S_j, _, _ = orc.scan(_bh(q), _bh(k), _bh(v[:, j:j + 1]), _bh(bpv[:, j]), _bh(lam),
                                      rule=DELTA, S0=S0[:, :, :, j:j + 1], lam_scaled=scaled)
            np.testing.assert_allclose(o[..., j], o_j[..., 0], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(S[..., j], S_j[..., 0], rtol=1e-12, atol=1e-13)
    for _ in range(200):
        S = rng.standard_normal((1, 1, dk, dv))
        xp = rng.standard_normal(dk)
        vt = rng.standard_normal(dv)
        bt = rng.uniform(0.01, 1.99, dv)
        lt = rng.uniform(0.0, 1.0)
        S1 = orc.step(rng.standard_normal((1, 1, dk)), rng.standard_normal((1, 1, dk)), vt[None, None],
                      bt[None, None], np.array([[lt]]), rule=PV, eps=0.0, S0=S,
                      xprev0=xp[None, None], has0=np.array([[1]]))[1]
        for j in range(dv):
            loss = lambda M: 0.5 * (vt[j] - M[:, j] @ xp) ** 2 + 0.5 * lt * M[:, j] @ M[:, j]
            assert loss(S1[0, 0]) <= loss(S[0, 0]) + 1e-12
    q = np.array([[0.0, 1.0], [1.0, 0.0]])
    k = np.array([[3.0, 4.0], [1.0, 1.0]])
    v = np.array([[7.0, 7.0], [10.0, 20.0]])
    beta = np.array([[0.3, 0.3], [1.0, 0.5]])
    S0 = np.array([[1.0, 2.0], [3.0, 4.0]])[None, None]
    o, S, _, _ = orc.scan(_bh(q), _bh(k), _bh(v), _bh(beta), _bh(np.array([0.0, 5.0])), rule=PV,
                          eps=0.0, S0=S0)
    np.testing.assert_allclose(S[0, 0], [[1 / 3, 26 / 15], [11 / 6, 53 / 15]], rtol=1e-14)
    np.testing.assert_allclose(o[0, 0], [[3.0, 4.0], [1 / 3, 26 / 15]], rtol=1e-14)


def pin_p24_backward(orc):
    """The backward pass (reading D21) against the forward oracle and closed forms.
    (a) Central finite differences (h = 1e-6) of L = sum(dO o) + sum(dS S_T) match every
        gradient (q, k, v, beta, lambda, S0, the carried key) for the delta, inner and
        additive rules, scalar and per-channel lambda, phi identity and elu+1, from a
        nonzero state with a carried key.
    (b) Linear attention (additive, gamma = beta = 1, S0 = 0, identity): brute-force sums
        dv_j = sum_{t>=j} (q_t . k_j) dO_t, dq_t = sum_{j<=t} k_j (v_j . dO_t),
        dk_j = sum_{t>=j} q_t (v_j . dO_t).
    (c) The delta rule's first token at a sequence start writes nothing, so the gradients of
        its beta and lambda are exactly zero.
    (d) With gate pre-activations (2 sigmoid or sigmoid for beta; softplus ridge or sigmoid
        retention for lambda), finite differences in the pre-activations match the
        gradients, scalar and per channel.
    (e) With QK normalisation (l2 and RMS), finite differences in the raw q, k and carried
        key match their gradients, every rule; and a key scaled by any c > 0 changes
        nothing, so its gradient is orthogonal to it.
    (f) With the scale-coupled ridge (lambda |x|^2), finite differences match the gradients
        of k, the carried key, beta and lambda, delta and inner rules, scalar and per
        channel.
    (g) The per-value-channel rule: finite differences match every gradient (q, k, v, the
        per-channel beta, lambda, S0, the carried key), plain, with elu+1, and with the
        scale-coupled ridge and pre-activated gates; with every beta_j equal it is the
        delta rule, and so are its gradients (beta's summed over j).
    (h) Normalised linear attention (additive, znorm): finite differences of
        L + sum(dz z_T) match every gradient (q, k, v, beta, gamma, S0 and the initial z),
        scalar and per-channel retention, positive identity features (raw or l2-normalised
        by the scan, which leaves z itself unscaled) and elu+1; and a sequence split over
        two calls, the second call's state gradient fed to the first as its (dS, dz),
        gives the one-call gradients."""
    rng = np.random.default_rng(42)
    T, dk, dv = 5, 3, 2
    for rule in (DELTA, INNER, ADD):
        for per_channel in (False, True):
            for phi_kind in ("identity", "elu1"):
                q, k = rng.standard_normal((1, 1, T, dk)), rng.standard_normal((1, 1, T, dk))
                v = rng.standard_normal((1, 1, T, dv))
                lshape = (1, 1, T, dk) if per_channel else (1, 1, T)
                if rule == ADD:
                    b, lam = rng.uniform(0.2, 1.5, (1, 1, T)), rng.uniform(0.6, 1.0, lshape)
                else:
                    b, lam = rng.uniform(0.2, 1.5, (1, 1, T)), rng.uniform(0.05, 0.5, lshape)
                dO, dS = rng.standard_normal((1, 1, T, dv)), rng.standard_normal((1, 1, dk, dv))
                S0, x0 = rng.standard_normal((1, 1, dk, dv)), rng.uniform(0.2, 1.0, (1, 1, dk))
                h0 = np.array([[1]])
                kw = dict(rule=rule, phi_kind=phi_kind, per_channel=per_channel, has0=h0)
                args = {"q": q, "k": k, "v": v, "beta": b, "lam": lam, "S0": S0, "xprev0": x0}

                def loss(a):
                    o, S, _, _ = orc.scan(a["q"], a["k"], a["v"], a["beta"], a["lam"], S0=a["S0"],
                                          xprev0=a["xprev0"], **kw)
                    return float(np.sum(o * dO) + np.sum(S * dS))

                gr = orc.scan_backward(q, k, v, b, lam, dO, dS, S0=S0, xprev0=x0, **kw)
                for name, arr in args.items():
                    for idx in np.ndindex(arr.shape):
                        a = dict(args)
                        ap, am = arr.copy(), arr.copy()
                        ap[idx] += 1e-6
                        am[idx] -= 1e-6
                        a[name] = ap
                        fp = loss(a)
                        a[name] = am
                        fd = (fp - loss(a)) / 2e-6
                        an = gr[name][idx]
                        assert abs(fd - an) <= 1e-6 * (1.0 + abs(an)), (rule, per_channel, phi_kind, name, idx, fd, an)
    q, k = rng.standard_normal((1, 1, 6, 4)), rng.standard_normal((1, 1, 6, 4))
    v, dO = rng.standard_normal((1, 1, 6, 3)), rng.standard_normal((1, 1, 6, 3))
    gr = orc.scan_backward(q, k, v, None, None, dO, rule=ADD)
    Q, K, V, D = q[0, 0], k[0, 0], v[0, 0], dO[0, 0]
    for j in range(6):
        np.testing.assert_allclose(gr["v"][0, 0, j], sum((Q[t] @ K[j]) * D[t] for t in range(j, 6)), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(gr["k"][0, 0, j], sum(Q[t] * (V[j] @ D[t]) for t in range(j, 6)), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(gr["q"][0, 0, j], sum(K[i] * (V[i] @ D[j]) for i in range(j + 1)), rtol=1e-12, atol=1e-12)
    b, lam = rng.uniform(0.2, 1.5, (1, 1, 6)), rng.uniform(0.05, 0.5, (1, 1, 6))
    gr = orc.scan_backward(q, k, v, b, lam, dO, rng.standard_normal((1, 1, 4, 3)), rule=DELTA,
                           S0=rng.standard_normal((1, 1, 4, 3)))
    assert gr["beta"][0, 0, 0] == 0.0 and gr["lam"][0, 0, 0] == 0.0
    for rule, bact in ((DELTA, "sigmoid2"), (INNER, "sigmoid"), (ADD, "sigmoid")):
        for per_channel in (False, True):
            T, dk, dv = 4, 3, 2
            q, k = rng.standard_normal((1, 1, T, dk)), rng.standard_normal((1, 1, T, dk))
            v = rng.standard_normal((1, 1, T, dv))
            zb = rng.standard_normal((1, 1, T))
            zl = rng.normal(-1.0 if rule != ADD else 2.0, 1.0, (1, 1, T, dk) if per_channel else (1, 1, T))
            dO, dS = rng.standard_normal((1, 1, T, dv)), rng.standard_normal((1, 1, dk, dv))
            S0, x0 = rng.standard_normal((1, 1, dk, dv)), rng.uniform(0.2, 1.0, (1, 1, dk))
            kw = dict(rule=rule, per_channel=per_channel, has0=np.array([[1]]), S0=S0, xprev0=x0,
                      beta_act=bact, lam_act=True)

            def loss(b, lam):
                o, S, _, _ = orc.scan(q, k, v, b, lam, **kw)
                return float(np.sum(o * dO) + np.sum(S * dS))

            gr = orc.scan_backward(q, k, v, zb, zl, dO, dS, **kw)
            for name, arr in (("beta", zb), ("lam", zl)):
                for idx in np.ndindex(arr.shape):
                    ap, am = arr.copy(), arr.copy()
                    ap[idx] += 1e-6
                    am[idx] -= 1e-6
                    fd = ((loss(ap, zl) - loss(am, zl)) if name == "beta" else (loss(zb, ap) - loss(zb, am))) / 2e-6
                    an = gr[name][idx]
                    assert abs(fd - an) <= 1e-6 * (1.0 + abs(an)), (rule, per_channel, name, idx, fd, an)
    for rule in (DELTA, INNER, ADD):
        for qk in ("l2", "rms"):
            T, dk, dv = 4, 3, 2
            q, k = rng.standard_normal((1, 1, T, dk)), rng.standard_normal((1, 1, T, dk))
            v = rng.standard_normal((1, 1, T, dv))
            b, lam = rng.uniform(0.2, 1.5, (1, 1, T)), rng.uniform(0.6, 1.0, (1, 1, T))
            dO, dS = rng.standard_normal((1, 1, T, dv)), rng.standard_normal((1, 1, dk, dv))
            S0, x0 = rng.standard_normal((1, 1, dk, dv)), rng.standard_normal((1, 1, dk))
            kw = dict(rule=rule, has0=np.array([[1]]), S0=S0, qk_norm=qk)
            args = {"q": q, "k": k, "xprev0": x0}

            def loss(a):
                o, S, _, _ = orc.scan(a["q"], a["k"], v, b, lam, xprev0=a["xprev0"], **kw)
                return float(np.sum(o * dO) + np.sum(S * dS))

            gr = orc.scan_backward(q, k, v, b, lam, dO, dS, xprev0=x0, **kw)
            for name, arr in args.items():
                if rule == ADD and name == "xprev0":
                    continue
                for idx in np.ndindex(arr.shape):
                    a = dict(args)
                    ap, am = arr.copy(), arr.copy()
                    ap[idx] += 1e-6
                    am[idx] -= 1e-6
                    a[name] = ap
                    fp = loss(a)
                    a[name] = am
                    fd = (fp - loss(a)) / 2e-6
                    an = gr[name][idx]
                    assert abs(fd - an) <= 1e-6 * (1.0 + abs(an)), (rule, qk, name, idx, fd, an)
            for name in ("q", "k"):
                dots = np.sum(gr[name] * args[name], axis=-1)
                assert np.all(np.abs(dots) <= 1e-12 * (1.0 + np.abs(gr[name]).sum())), (rule, qk, name)
    for rule in (DELTA, INNER):
        for per_channel in (False, True):
            T, dk, dv = 4, 3, 2
            q, k = rng.standard_normal((1, 1, T, dk)), rng.standard_normal((1, 1, T, dk))
            v = rng.standard_normal((1, 1, T, dv))
            b = rng.uniform(0.2, 1.5, (1, 1, T))
            lam = rng.uniform(0.05, 0.5, (1, 1, T, dk) if per_channel else (1, 1, T))
            dO, dS = rng.standard_normal((1, 1, T, dv)), rng.standard_normal((1, 1, dk, dv))
            S0, x0 = rng.standard_normal((1, 1, dk, dv)), rng.standard_normal((1, 1, dk))
            kw = dict(rule=rule, per_channel=per_channel, has0=np.array([[1]]), S0=S0,
                      lam_scaled=True)
            args = {"k": k, "xprev0": x0, "beta": b, "lam": lam}

            def loss(a):
                o, S, _, _ = orc.scan(q, a["k"], v, a["beta"], a["lam"], xprev0=a["xprev0"], **kw)
                return float(np.sum(o * dO) + np.sum(S * dS))

            gr = orc.scan_backward(q, k, v, b, lam, dO, dS, xprev0=x0, **kw)
            for name, arr in args.items():
                for idx in np.ndindex(arr.shape):
                    a = dict(args)
                    ap, am = arr.copy(), arr.copy()
                    ap[idx] += 1e-6
                    am[idx] -= 1e-6
                    a[name] = ap
                    fp = loss(a)
                    a[name] = am
                    fd = (fp - loss(a)) / 2e-6
                    an = gr[name][idx]
                    assert abs(fd - an) <= 1e-6 * (1.0 + abs(an)), (rule, per_channel, name, idx, fd, an)

    PV = orc.RULE_DELTA_PV
    for variant in ("plain", "elu1", "scaled_gates"):
        T, dk, dv = 4, 3, 2
        q, k = rng.standard_normal((1, 1, T, dk)), rng.standard_normal((1, 1, T, dk))
        v = rng.standard_normal((1, 1, T, dv))
        if variant == "scaled_gates":
            b, lam = rng.standard_normal((1, 1, T, dv)), rng.normal(-1.0, 1.0, (1, 1, T))
        else:
            b, lam = rng.uniform(0.2, 1.5, (1, 1, T, dv)), rng.uniform(0.05, 0.5, (1, 1, T))
        dO, dS = rng.standard_normal((1, 1, T, dv)), rng.standard_normal((1, 1, dk, dv))
        S0, x0 = rng.standard_normal((1, 1, dk, dv)), rng.uniform(0.2, 1.0, (1, 1, dk))
        kw = dict(rule=PV, has0=np.array([[1]]), phi_kind="elu1" if variant == "elu1" else "identity")
        if variant == "scaled_gates":
            kw.update(lam_scaled=True, beta_act="sigmoid2", lam_act=True)
        args = {"q": q, "k": k, "v": v, "beta": b, "lam": lam, "S0": S0, "xprev0": x0}

        def loss(a):
            o, S, _, _ = orc.scan(a["q"], a["k"], a["v"], a["beta"], a["lam"], S0=a["S0"],
                                  xprev0=a["xprev0"], **kw)
            return float(np.sum(o * dO) + np.sum(S * dS))

        gr = orc.scan_backward(q, k, v, b, lam, dO, dS, S0=S0, xprev0=x0, **kw)
        for name, arr in args.items():
            for idx in np.ndindex(arr.shape):
                a = dict(args)
                ap, am = arr.copy(), arr.copy()
                ap[idx] += 1e-6
                am[idx] -= 1e-6
                a[name] = ap
                fp = loss(a)
                a[name] = am
                fd = (fp - loss(a)) / 2e-6
                an = gr[name][idx]
                assert abs(fd - an) <= 1e-6 * (1.0 + abs(an)), (variant, name, idx, fd, an)
    # equal steps on every value channel: the delta rule
    b1 = rng.uniform(0.2, 1.5, (1, 1, T))
    bpv = np.repeat(b1[..., None], dv, axis=-1)
    g_pv = orc.scan_backward(q, k, v, bpv, lam, dO, dS, rule=PV, S0=S0, xprev0=x0, has0=np.array([[1]]))
    g_d = orc.scan_backward(q, k, v, b1, lam, dO, dS, rule=DELTA, S0=S0, xprev0=x0, has0=np.array([[1]]))
    for name in ("q", "k", "v", "lam", "S0", "xprev0"):
        np.testing.assert_allclose(g_pv[name], g_d[name], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g_pv["beta"].sum(axis=-1), g_d["beta"], rtol=1e-12, atol=1e-12)

    for per_channel in (False, True):
        for phi_kind in ("identity", "elu1", "identity_l2"):
            T, dk, dv = 4, 3, 2
            q, k = rng.standard_normal((1, 1, T, dk)), rng.standard_normal((1, 1, T, dk))
            if phi_kind != "elu1":
                q, k = np.abs(q) + 0.1, np.abs(k) + 0.1
            v = rng.standard_normal((1, 1, T, dv))
            b = rng.uniform(0.2, 1.5, (1, 1, T))
            lam = rng.uniform(0.6, 1.0, (1, 1, T, dk) if per_channel else (1, 1, T))
            dO, dS = rng.standard_normal((1, 1, T, dv)), rng.standard_normal((1, 1, dk, dv))
            S0, z0 = rng.standard_normal((1, 1, dk, dv)), rng.uniform(0.2, 1.0, (1, 1, dk))
            dz = rng.standard_normal((1, 1, dk))
            kw = dict(rule=ADD, per_channel=per_channel, znorm=True,
                      phi_kind="elu1" if phi_kind == "elu1" else "identity",
                      qk_norm="l2" if phi_kind == "identity_l2" else None)
            args = {"q": q, "k": k, "v": v, "beta": b, "lam": lam, "S0": S0, "xprev0": z0}

            def loss(a):
                o, S, zT, _ = orc.scan(a["q"], a["k"], a["v"], a["beta"], a["lam"], S0=a["S0"],
                                       xprev0=a["xprev0"], **kw)
                return float(np.sum(o * dO) + np.sum(S * dS) + np.sum(zT * dz))

            gr = orc.scan_backward(q, k, v, b, lam, dO, dS, S0=S0, xprev0=z0, dz=dz, **kw)
            # two calls: the second call's gradients of its initial S and z are the first
            # call's (dS, dz)
            T1 = 2
            cut = lambda x, a, e: x[:, :, a:e]
            _, S1, z1, h1 = orc.scan(cut(q, 0, T1), cut(k, 0, T1), cut(v, 0, T1), cut(b, 0, T1),
                                     cut(lam, 0, T1), S0=S0, xprev0=z0, **kw)
            g2 = orc.scan_backward(cut(q, T1, T), cut(k, T1, T), cut(v, T1, T), cut(b, T1, T),
                                   cut(lam, T1, T), cut(dO, T1, T), dS, S0=S1, xprev0=z1,
                                   has0=h1, dz=dz, **kw)
            g1 = orc.scan_backward(cut(q, 0, T1), cut(k, 0, T1), cut(v, 0, T1), cut(b, 0, T1),
                                   cut(lam, 0, T1), cut(dO, 0, T1), g2["S0"], S0=S0, xprev0=z0,
                                   dz=g2["xprev0"], **kw)
            for name in ("q", "k", "v", "beta", "lam"):
                both = np.concatenate([g1[name], g2[name]], axis=2)
                np.testing.assert_allclose(both, gr[name], rtol=1e-10, atol=1e-12)
            for name in ("S0", "xprev0"):
                np.testing.assert_allclose(g1[name], gr[name], rtol=1e-10, atol=1e-12)
            for name, arr in args.items():
                for idx in np.ndindex(arr.shape):
                    a = dict(args)
                    ap, am = arr.copy(), arr.copy()
                    ap[idx] += 1e-6
                    am[idx] -= 1e-6
                    a[name] = ap
                    fp = loss(a)
                    a[name] = am
                    fd = (fp - loss(a)) / 2e-6
                    an = gr[name][idx]
                    assert abs(fd - an) <= 1e-6 * (1.0 + abs(an)), (per_channel, phi_kind, name, idx, fd, an)


ALL_PINS = [
    pin_p1_outer_product_store,
    pin_p2_quadratic_form,
    pin_p2_decayed_quadratic_form,
    pin_p3_first_step_noop,
    pin_p4_nlms_rewrite,
    pin_p5_orthonormal_recall,
    pin_p6_descent_lemma,
    pin_p7_zero_beta,
    pin_p8_per_channel_equal,
    pin_p9_hand_delta,
    pin_p9_hand_additive,
    pin_p10_state_carry,
    pin_p11_interference_ratio,
    pin_p12_min_norm_store,
    pin_p13_inner_hebbian_sum,
    pin_p14_inner_decayed_sum,
    pin_p15_inner_gradient_step,
    pin_p16_inner_first_step_noop,
    pin_p17_inner_is_shifted_linear_attention,
    pin_p9_hand_inner,
    pin_p18_qk_norm_is_the_rule_on_normalised_inputs,
    pin_p19_qk_norm_scale_invariance,
    pin_p20_gate_preactivations,
    pin_p21_normalised_linear_attention,
    pin_p22_scale_coupled_ridge,
    pin_p23_per_value_channel_rule,
    pin_p24_backward,
    pin_relerr_metric,
]
