"""Seeded synthetic workloads for the fast-weight scan.

This module only draws random inputs. It holds none of the scan's arithmetic,
imports nothing else from this package, and is the one piece of code that the
GPU path's tests/benchmark and the CPU oracle both use.

Every floating-point array is returned as float32 whose values are exactly the
values the kernels consume: for bf16 workloads each value is already rounded to
bf16 (round to nearest even), so converting it to torch.bfloat16 is exact and
the oracle reads the very same numbers in float64.

Recipes (the names match the workload table of the design document):

  delta_f32_small   B=1 H=1 T=256 d=64, fp32, delta rule, phi = identity.
                    q,k,v ~ N(0,1); q,k L2-normalised per token;
                    beta = sigmoid(N(0,1)); lambda = 0.01; eps = 1e-6; S0 = 0.
  delta_bf16        B=4 H=8 T=4096 d=128, bf16 q,k,v, delta rule.
                    q,k,v ~ N(0,1), q,k L2-normalised (fp32) then rounded;
                    beta = 2*sigmoid(N(0,1)); lambda = softplus(N(-4,1)) per token
                    per head; S0 = 0.
  delta_bf16_h16    the throughput workload: as delta_bf16 with H=16.
  additive_bf16     B=2 H=16 T=16384 d=128, bf16, additive write, phi = elu+1.
                    q,k,v ~ N(0,1) (not normalised); gamma = sigmoid(N(3,0.5));
                    beta = 1 (no write scale); S0 = 0.
  delta_long_pc     B=1 H=8 T=131072 d=128, bf16, delta rule, per-key-channel
                    lambda = softplus(N(-5,1)) of shape [B,H,T,dk];
                    beta = sigmoid(N(0,1)); S0 = 0.
  inner_bf16        B=4 H=8 T=4096 d=128, bf16, inner-product rule (shifted pair,
                    normalised step, the target written in place of the residual);
                    delta_bf16's distributions (no workload on the pages fixes them).
  inner_f32_small   as delta_f32_small with the inner-product rule.
  delta_bf16_h16_qknorm  as delta_bf16_h16 with raw q, k ~ N(0,1) (not normalised, then
                    rounded) that the scan normalises to unit length itself.
  decode            B=256 H=32 d=128, 1000 single-token steps (delta rule).
                    S0 ~ N(0, 0.02) fp32 with no previous key; per step
                    q,k,v ~ N(0,1) bf16 with q,k normalised; beta = sigmoid(N(0,1));
                    lambda = 0.01.

Draw order for a scan: q, k, v, then the beta pre-activation, then the lambda /
gamma pre-activation, then S0 (only when the recipe has one). N(mu, s): s is the
standard deviation. Decode steps draw from default_rng([seed, 1 + step]) so a
single step can be regenerated on its own; S0 comes from default_rng([seed, 0]).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

RULE_DELTA = 0
RULE_ADDITIVE = 1
RULE_INNER = 2
RULE_DELTA_PV = 3
PHI_IDENTITY = "identity"
PHI_ELU1 = "elu1"


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), returned as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    out = (rounded << 16).astype(np.uint32)
    return out.view(np.float32).reshape(x.shape)


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True))
    return (x / np.maximum(n, np.float32(1e-12))).astype(np.float32)


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-z.astype(np.float64)))).astype(np.float32)


def _softplus(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float64)
    return (np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))).astype(np.float32)


@dataclasses.dataclass
class ScanInputs:
    """One synthetic scan problem. Arrays are float32 (bf16-exact when dtype == 'bf16')."""
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str               # 'bf16' or 'f32': the storage type of q, k, v and out
    rule: int                # RULE_DELTA, RULE_ADDITIVE, RULE_INNER or RULE_DELTA_PV
    phi: str                 # PHI_IDENTITY or PHI_ELU1
    per_channel: bool        # lambda is [B,H,T,dk] instead of [B,H,T]
    eps: float
    q: np.ndarray            # [B,H,T,dk]
    k: np.ndarray            # [B,H,T,dk]
    v: np.ndarray            # [B,H,T,dv]
    beta: Optional[np.ndarray]   # [B,H,T] float32 ([B,H,T,dv] for RULE_DELTA_PV), or None
                                 # (= 1, additive only)
    lam: Optional[np.ndarray]    # [B,H,T] or [B,H,T,dk] float32, or None
    S0: Optional[np.ndarray] = None        # [B,H,dk,dv] float32 or None (= 0)
    xprev0: Optional[np.ndarray] = None    # [B,H,dk] float32 or None
    has0: Optional[np.ndarray] = None      # [B,H] int32 or None
    qk_norm: Optional[str] = None          # None, 'l2' or 'rms': q, k are raw and the scan
                                           # normalises them (the library's QK flags)
    beta_pre: Optional[np.ndarray] = None  # the pre-activations the gates were drawn from
    lam_pre: Optional[np.ndarray] = None
    beta_act: Optional[str] = None         # how beta follows from beta_pre: 'sigmoid', 'sigmoid2'
    lam_act: bool = False                  # lam = softplus(lam_pre) (or sigmoid for gamma)
    gates_pre: bool = False                # hand the library the pre-activations (its gate flags)
    znorm: bool = False                    # normalised linear attention (additive rule): the
                                           # read is divided by z . q, z the state's x_prev slot
    lam_scaled: bool = False               # lam is a base ridge, times the written key's energy

    @property
    def tokens(self) -> int:
        return self.B * self.T


def _normal(rng, shape, mean=0.0, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def make_scan(*, B, H, T, dk, dv, dtype="bf16", rule=RULE_DELTA, phi=PHI_IDENTITY,
              normalise_qk=True, beta_kind="sigmoid", lam_kind="const",
              lam_const=0.01, lam_mu=-4.0, per_channel=False, gamma_mu=3.0,
              gamma_sd=0.5, eps=1e-6, s0_std=None, seed=0, name="custom",
              qk_norm=None, qk_positive=False, znorm=False, lam_scaled=False) -> ScanInputs:
    """Draw one scan problem.

    beta_kind: 'sigmoid' (sigmoid(N(0,1))), 'two_sigmoid' (2*sigmoid(N(0,1))),
               'one' (beta = None: unit write scale, additive only), or a float
               (every beta equal to it).
    lam_kind:  'const' (lam_const everywhere), 'softplus' (softplus(N(lam_mu,1))),
               'gamma' (sigmoid(N(gamma_mu, gamma_sd)), the additive retention),
               'none' (lam = None).
    qk_positive: q, k drawn as |N(0,1)| (positive features for the identity map, so that
               the normaliser of znorm stays positive).
    znorm:     normalised linear attention; with s0_std the initial normaliser z0 (the
               x_prev slot) is drawn as |N(0,1)| times the initial state's scale.
    """
    rng = np.random.default_rng(seed)
    q = _normal(rng, (B, H, T, dk))
    k = _normal(rng, (B, H, T, dk))
    v = _normal(rng, (B, H, T, dv))
    if qk_positive:
        q, k = np.abs(q), np.abs(k)
    if normalise_qk:
        q = _l2_normalise(q)
        k = _l2_normalise(k)
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    elif dtype != "f32":
        raise ValueError(dtype)

    beta_pre = lam_pre = beta_act = None
    lam_act = False
    bshape = (B, H, T, dv) if rule == RULE_DELTA_PV else (B, H, T)
    if beta_kind == "sigmoid":
        beta_pre = _normal(rng, bshape)
        beta, beta_act = _sigmoid(beta_pre), "sigmoid"
    elif beta_kind == "two_sigmoid":
        beta_pre = _normal(rng, bshape)
        beta, beta_act = (2.0 * _sigmoid(beta_pre)).astype(np.float32), "sigmoid2"
    elif beta_kind == "one":
        beta = None
    else:
        beta = np.full(bshape, float(beta_kind), dtype=np.float32)

    lam_shape = (B, H, T, dk) if per_channel else (B, H, T)
    if lam_kind == "const":
        lam = np.full(lam_shape, lam_const, dtype=np.float32)
    elif lam_kind == "softplus":
        lam_pre = _normal(rng, lam_shape, mean=lam_mu)
        lam, lam_act = _softplus(lam_pre), True
    elif lam_kind == "gamma":
        lam_pre = _normal(rng, lam_shape, mean=gamma_mu, std=gamma_sd)
        lam, lam_act = _sigmoid(lam_pre), True
    elif lam_kind == "none":
        lam = None
    else:
        raise ValueError(lam_kind)

    S0 = xprev0 = None
    if s0_std is not None:
        S0 = _normal(rng, (B, H, dk, dv), std=s0_std)
        if znorm:
            xprev0 = np.abs(_normal(rng, (B, H, dk), std=s0_std))
    return ScanInputs(name=name, B=B, H=H, T=T, dk=dk, dv=dv, dtype=dtype, rule=rule,
                      phi=phi, per_channel=per_channel, eps=eps, q=q, k=k, v=v,
                      beta=beta, lam=lam, S0=S0, xprev0=xprev0, qk_norm=qk_norm,
                      beta_pre=beta_pre, lam_pre=lam_pre, beta_act=beta_act, lam_act=lam_act,
                      znorm=znorm, lam_scaled=lam_scaled)


def delta_f32_small(seed=0, T=256):
    return make_scan(B=1, H=1, T=T, dk=64, dv=64, dtype="f32", beta_kind="sigmoid",
                     lam_kind="const", lam_const=0.01, seed=seed, name="delta_f32_small")


def delta_bf16(seed=0, B=4, H=8, T=4096, d=128):
    return make_scan(B=B, H=H, T=T, dk=d, dv=d, dtype="bf16", beta_kind="two_sigmoid",
                     lam_kind="softplus", lam_mu=-4.0, seed=seed, name="delta_bf16")


def delta_bf16_h16(seed=0, B=4, T=4096, d=128):
    w = delta_bf16(seed=seed, B=B, H=16, T=T, d=d)
    w.name = "delta_bf16_h16"
    return w


def additive_bf16(seed=0, B=2, H=16, T=16384, d=128):
    return make_scan(B=B, H=H, T=T, dk=d, dv=d, dtype="bf16", rule=RULE_ADDITIVE,
                     phi=PHI_ELU1, normalise_qk=False, beta_kind="one", lam_kind="gamma",
                     gamma_mu=3.0, gamma_sd=0.5, seed=seed, name="additive_bf16")


def delta_long_pc(seed=0, B=1, H=8, T=131072, d=128):
    return make_scan(B=B, H=H, T=T, dk=d, dv=d, dtype="bf16", beta_kind="sigmoid",
                     lam_kind="softplus", lam_mu=-5.0, per_channel=True, seed=seed,
                     name="delta_long_pc")


def delta_bf16_h16_qknorm(seed=0, B=4, T=4096, d=128):
    """The throughput workload with raw q, k ~ N(0,1) bf16, normalised by the scan itself
    (unit length): the same gates as delta_bf16_h16."""
    return make_scan(B=B, H=16, T=T, dk=d, dv=d, dtype="bf16", beta_kind="two_sigmoid",
                     lam_kind="softplus", lam_mu=-4.0, normalise_qk=False, qk_norm="l2",
                     seed=seed, name="delta_bf16_h16_qknorm")


def inner_bf16(seed=0, B=4, H=8, T=4096, d=128):
    return make_scan(B=B, H=H, T=T, dk=d, dv=d, dtype="bf16", rule=RULE_INNER,
                     beta_kind="two_sigmoid", lam_kind="softplus", lam_mu=-4.0, seed=seed,
                     name="inner_bf16")


def additive_znorm_bf16(seed=0, B=2, H=16, T=16384, d=128):
    """additive_bf16 with the normaliser: linear attention with elu+1 features and a
    retention gate, each read divided by z . phi(q)."""
    w = additive_bf16(seed=seed, B=B, H=H, T=T, d=d)
    w.znorm, w.name = True, "additive_znorm_bf16"
    return w


def delta_pv_bf16_h16(seed=0, B=4, T=4096, d=128):
    """The throughput workload's shape and distributions with one step size per value
    channel (Falcon-2): beta = 2 sigmoid(N(0,1)) drawn per (token, value channel)."""
    return make_scan(B=B, H=16, T=T, dk=d, dv=d, dtype="bf16", rule=RULE_DELTA_PV,
                     beta_kind="two_sigmoid", lam_kind="softplus", lam_mu=-4.0, seed=seed,
                     name="delta_pv_bf16_h16")


def inner_f32_small(seed=0, T=256):
    return make_scan(B=1, H=1, T=T, dk=64, dv=64, dtype="f32", rule=RULE_INNER,
                     beta_kind="sigmoid", lam_kind="const", lam_const=0.01, seed=seed,
                     name="inner_f32_small")


# ---------------------------------------------------------------- decode (one token per step)

@dataclasses.dataclass
class DecodeStep:
    q: np.ndarray      # [B,H,dk] float32 (bf16-exact)
    k: np.ndarray
    v: np.ndarray      # [B,H,dv]
    beta: np.ndarray   # [B,H]
    lam: np.ndarray    # [B,H]


def decode_state0(seed=0, B=256, H=32, d=128, std=0.02) -> np.ndarray:
    """S0 ~ N(0, std) of shape [B,H,d,d], float32."""
    rng = np.random.default_rng([seed, 0])
    return _normal(rng, (B, H, d, d), std=std)


def decode_step(seed, step, B=256, H=32, d=128, lam_const=0.01) -> DecodeStep:
    rng = np.random.default_rng([seed, 1 + step])
    q = round_to_bf16(_l2_normalise(_normal(rng, (B, H, d))))
    k = round_to_bf16(_l2_normalise(_normal(rng, (B, H, d))))
    v = round_to_bf16(_normal(rng, (B, H, d)))
    beta = _sigmoid(_normal(rng, (B, H)))
    lam = np.full((B, H), lam_const, dtype=np.float32)
    return DecodeStep(q=q, k=k, v=v, beta=beta, lam=lam)


SCAN_WORKLOADS = {
    "delta_f32_small": delta_f32_small,
    "delta_bf16": delta_bf16,
    "delta_bf16_h16": delta_bf16_h16,
    "additive_bf16": additive_bf16,
    "delta_long_pc": delta_long_pc,
    "inner_bf16": inner_bf16,
    "delta_bf16_h16_qknorm": delta_bf16_h16_qknorm,
    "inner_f32_small": inner_f32_small,
    "additive_znorm_bf16": additive_znorm_bf16,
    "delta_pv_bf16_h16": delta_pv_bf16_h16,
}
