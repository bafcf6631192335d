"""The segment-parallel form of the scan, checked on the fp64 oracle (CPU).

The library cuts a few-head, long sequence into P segments that run as separate heads:
a local pass from the zero state (giving each segment's own state B_p), a transition pass
from the identity with zero values (giving A_p of the segment's map S -> A_p S + B_p),
a serial chain S_start(p+1) = A_p S_start(p) + B_p from S_start(0), the caller's state,
and one pass over the segments from their true start states that forms the outputs. The
write of every rule is affine in S ("Fast Weight Attention for Continual Learning"
reading notes, sections 3.2, 4.2 and 4.3; "attention is also an FFN", section 3.2), so
this equals the sequential scan up to rounding. Here the decomposition itself is run on
the oracle and compared with one sequential scan."""
import numpy as np
import pytest

from linear_attention_scan_amd import fwmem as F
from linear_attention_scan_amd import workloads as wl
from oracle import fwmem_oracle as orc


def _segmented(w, P, S0=None, x0=None, h0=None):
    B, H, T, dk = w.q.shape
    dv = w.v.shape[-1]
    L = T // P
    N = B * H
    r = lambda a, tail: None if a is None else a.reshape((N * P, L) + a.shape[3:] if tail else (N * P, L))
    q, k, v = (a.reshape(N * P, L, a.shape[-1]) for a in (w.q, w.k, w.v))
    beta = None if w.beta is None else w.beta.reshape(N * P, L)
    lam = None if w.lam is None else (w.lam.reshape(N * P, L, dk) if w.per_channel else w.lam.reshape(N * P, L))
    kk = w.k.reshape(N, T, dk)
    # virtual start states: carried key = the previous segment's last key
    xv = np.zeros((N, P, dk))
    hv = np.ones((N, P), dtype=np.int32)
    for p in range(1, P):
        xv[:, p] = orc.phi(kk[:, p * L - 1], w.phi)
    hv[:, 0] = 0 if h0 is None else h0.reshape(N)
    if x0 is not None:
        xv[:, 0] = x0.reshape(N, dk)
    Sa = np.broadcast_to(np.eye(dk), (N, P, dk, dk)).copy()
    kw = dict(rule=w.rule, phi_kind=w.phi, eps=w.eps, per_channel=w.per_channel, qk_norm=w.qk_norm)
    sh = lambda a: a[:, None] if a is not None else None
    xs, hs = xv.reshape(N * P, 1, dk), hv.reshape(N * P, 1)
    _, B1, _, _ = orc.scan(sh(q), sh(k), sh(v), sh(beta), sh(lam), S0=np.zeros((N * P, 1, dk, dv)),
                           xprev0=xs, has0=hs, **kw)
    _, A1, _, _ = orc.scan(sh(q), sh(k), sh(np.zeros((N * P, L, dk))), sh(beta), sh(lam),
                           S0=Sa.reshape(N * P, 1, dk, dk), xprev0=xs, has0=hs, **kw)
    A1, B1 = A1.reshape(N, P, dk, dk), B1.reshape(N, P, dk, dv)
    starts = np.zeros((N, P, dk, dv))
    S = np.zeros((N, dk, dv)) if S0 is None else S0.reshape(N, dk, dv).copy()
    for p in range(P):
        starts[:, p] = S
        S = np.einsum("nij,njv->niv", A1[:, p], S) + B1[:, p]
    o, _, _, _ = orc.scan(sh(q), sh(k), sh(v), sh(beta), sh(lam), S0=starts.reshape(N * P, 1, dk, dv),
                          xprev0=xs, has0=hs, **kw)
    return o.reshape(B, H, T, dv), S.reshape(B, H, dk, dv)


@pytest.mark.parametrize("name,P", [("delta", 4), ("inner", 8), ("additive", 4), ("delta_pc", 4), ("delta_qk", 4)])
def test_segmented_scan_equals_sequential(name, P):
    mk = dict(B=1, H=2, T=96, dk=6, dv=5, dtype="f32", seed=len(name) + P)
    if name == "delta":
        w = wl.make_scan(beta_kind="two_sigmoid", lam_kind="softplus", **mk)
    elif name == "inner":
        w = wl.make_scan(rule=wl.RULE_INNER, beta_kind="two_sigmoid", lam_kind="softplus", **mk)
    elif name == "additive":
        w = wl.make_scan(rule=wl.RULE_ADDITIVE, phi=wl.PHI_ELU1, normalise_qk=False, beta_kind="sigmoid",
                         lam_kind="gamma", **mk)
    elif name == "delta_pc":
        w = wl.make_scan(beta_kind="sigmoid", lam_kind="softplus", lam_mu=-2.0, per_channel=True, **mk)
    else:
        w = wl.make_scan(beta_kind="two_sigmoid", lam_kind="softplus", normalise_qk=False, qk_norm="rms", **mk)
    rng = np.random.default_rng(3)
    S0 = rng.standard_normal((1, 2, 6, 5)) * 0.3
    x0 = rng.standard_normal((1, 2, 6))
    h0 = np.array([[1, 0]], dtype=np.int32)
    o_ref, S_ref, _, _ = orc.scan(w.q, w.k, w.v, w.beta, w.lam, rule=w.rule, phi_kind=w.phi, eps=w.eps,
                                  per_channel=w.per_channel, qk_norm=w.qk_norm, S0=S0, xprev0=x0, has0=h0)
    o, S = _segmented(w, P, S0=S0, x0=x0, h0=h0)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-10 * np.abs(o_ref).max())
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-10 * np.abs(S_ref).max())


def test_workspace_grows_only_for_segmented_shapes():
    """The library segments only when the propagate grid would leave most of the GPU idle:
    the T = 131072, 8-head workload is segmented (P = 32 on bf16 inputs: the extra
    workspace holds the virtual start and end states of the local and transition passes
    of 256 virtual heads), the 64-head throughput workload is not."""
    def ws(B, H, T, d, dtype, flags):
        return F.workspace_bytes(F.shape(B, H, T, d, d, dtype), F.mode(0, flags, 1e-6, 0))
    rec = lambda BH, T, per: BH * (T // 64) * per
    per_split = ws(1, 1, 64, 128, F.BF16, 0)
    assert ws(4, 16, 4096, 128, F.BF16, 0) == -(-rec(64, 4096, per_split) // 256) * 256
    long_pc = ws(1, 8, 131072, 128, F.BF16, F.LAMBDA_PER_CHANNEL)
    per_gen = ws(1, 1, 64, 128, F.BF16, F.LAMBDA_PER_CHANNEL)
    vh = 8 * 32
    state = lambda n: vh * (128 * n + 128 + 1) * 4  # S [dk][n], x_prev [dk], has_prev
    assert long_pc >= rec(8, 131072, per_gen) + 2 * state(128) + 2 * state(128)
    # bf16 output disables the segmented form
    assert ws(1, 8, 131072, 128, F.BF16, F.LAMBDA_PER_CHANNEL | F.OUT_BF16) == \
        -(-rec(8, 131072, per_gen) // 256) * 256
