"""GPU parity of the fused additive scan (elu+1 features, scalar retention, bf16 inputs;
one kernel per head, no prep records) against the fp64 oracle.

Every operand that is not an exact bf16 input is carried as a bf16 hi + lo pair, so the
kernel keeps about 16 bits of each factor: the bound here is 1e-3 of rms (the bf16-input
bound is 2e-2). Cases span several 64-token chunks with a ragged tail, every head-size
pair, optional write scales, raw retentions with negative and zero values, a carried
state across two calls, bf16 output, large magnitudes and the segmented path."""
import numpy as np
import pytest

from linear_attention_scan_amd import fwmem as F
from linear_attention_scan_amd import workloads as wl
from oracle import fwmem_oracle as orc
from tests.gpu_helpers import check_scan, gpu_scan, oracle_scan, say, state_np

pytestmark = pytest.mark.gpu

TOL_SPLIT = 1e-3


def additive_elu(B, H, T, dk=128, dv=128, beta_kind="one", seed=0, name="additive elu"):
    return wl.make_scan(B=B, H=H, T=T, dk=dk, dv=dv, dtype="bf16", rule=wl.RULE_ADDITIVE,
                        phi=wl.PHI_ELU1, normalise_qk=False, beta_kind=beta_kind,
                        lam_kind="gamma", gamma_mu=3.0, gamma_sd=0.5, seed=seed, name=name)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("beta_kind", ["one", "sigmoid"])
def test_fused_additive_dims(dk, dv, beta_kind):
    w = additive_elu(2, 3, 333, dk, dv, beta_kind, seed=3 * dk + dv,
                     name=f"fused additive {dk}x{dv} beta={beta_kind}")
    check_scan(w, tol=TOL_SPLIT)


@pytest.mark.parametrize("T", [1, 5, 63, 64, 65, 128, 191])
def test_fused_additive_short(T):
    check_scan(additive_elu(1, 2, T, seed=100 + T, name=f"fused additive T={T}"), tol=TOL_SPLIT)


def test_fused_additive_raw_retention_signs():
    """Retentions passed as given (no activation), drawn in [-1, 1] with exact zeros: the
    decay products carry a sign parity, and a zero retention clears the state."""
    w = additive_elu(2, 2, 300, seed=21, name="fused additive raw retention")
    rng = np.random.default_rng(22)
    lam = rng.uniform(-1.0, 1.0, size=(2, 2, 300)).astype(np.float32)
    lam[:, :, ::37] = 0.0
    lam[:, :, 5::11] = np.abs(lam[:, :, 5::11]) ** 0.05  # near 1: long memory between the zeros
    w.lam, w.lam_pre, w.lam_act = lam, None, False
    w.S0 = (rng.standard_normal((2, 2, 128, 128)) * 0.2).astype(np.float32)
    check_scan(w, tol=TOL_SPLIT)


def test_fused_additive_carries_state():
    """scan(1..T1) then scan(T1+1..T) from the carried state, in place, equals one scan."""
    w = additive_elu(2, 2, 330, beta_kind="sigmoid", seed=23, name="fused additive split")
    T1 = 137
    say("[scan] fused additive, two calls with the state carried in place")
    o1, st = gpu_scan(w, t_slice=slice(0, T1))
    o2, st = gpu_scan(w, t_slice=slice(T1, None), S_in=st, S_out=st)
    o_ref, S_ref, x_ref, _ = oracle_scan(w)
    S, x, h = state_np(st)
    eo = orc.relerr(np.concatenate([o1, o2], axis=2), o_ref)
    eS = orc.relerr(S, S_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e}")
    assert eo <= TOL_SPLIT and eS <= TOL_SPLIT
    np.testing.assert_allclose(x, x_ref, rtol=4e-6, atol=1e-30)
    assert np.all(h == 1)


def test_fused_additive_out_bf16_is_rounded_fp32():
    import torch
    w = additive_elu(1, 2, 200, seed=24, name="fused additive out bf16")
    o32, _ = gpu_scan(w)
    o16, _ = gpu_scan(w, extra_flags=F.OUT_BF16)
    want = torch.from_numpy(o32.astype(np.float32)).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(o16.astype(np.float32), want)


def test_fused_additive_large_magnitudes():
    """|q|, |k| ~ 1e3 and |v| ~ 1e5: split operands keep fp32's exponent range."""
    w = additive_elu(1, 2, 200, seed=25, name="fused additive large")
    w.q = wl.round_to_bf16(w.q * 1e3)
    w.k = wl.round_to_bf16(w.k * 1e3)
    w.v = wl.round_to_bf16(w.v * 1e5)
    check_scan(w, tol=TOL_SPLIT)


def test_fused_additive_segmented():
    """Few heads on a long sequence: segment states first, the combine, then one fused
    pass per segment from its true start state."""
    w = additive_elu(1, 2, 8192, beta_kind="sigmoid", seed=26, name="fused additive segmented")
    rng = np.random.default_rng(27)
    w.S0 = (rng.standard_normal((1, 2, 128, 128)) * 0.1).astype(np.float32)
    check_scan(w, tol=TOL_SPLIT)


def test_fused_additive_repeatable():
    w = additive_elu(1, 2, 500, seed=28, name="fused additive repeat")
    a, sa = gpu_scan(w)
    b, sb = gpu_scan(w)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(state_np(sa)[0], state_np(sb)[0])


# ---- the normaliser carried by the fused kernel (z_t . phi(q_t) + eps divides each read)

def additive_elu_z(B, H, T, dk=128, dv=128, seed=0, **kw):
    w = additive_elu(B, H, T, dk, dv, kw.pop("beta_kind", "one"), seed=seed,
                     name=f"fused additive znorm {dk}x{dv} T={T}")
    w.znorm = True
    for k, v in kw.items():
        setattr(w, k, v)
    return w


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_fused_znorm_dims(dk, dv):
    check_scan(additive_elu_z(2, 2, 333, dk, dv, seed=40 + dk + dv, beta_kind="sigmoid"), tol=TOL_SPLIT)


@pytest.mark.parametrize("T", [1, 63, 65, 200])
def test_fused_znorm_short(T):
    check_scan(additive_elu_z(1, 2, T, seed=50 + T), tol=TOL_SPLIT)


def test_fused_znorm_carried_state_in_place():
    """Nonzero S0 and z0 (the key slot), the state updated in place."""
    from tests.gpu_helpers import make_state
    w = additive_elu_z(1, 2, 450, seed=60)
    rng = np.random.default_rng(61)
    w.S0 = (rng.standard_normal((1, 2, 128, 128)) * 0.05).astype(np.float32)
    w.xprev0 = np.abs(rng.standard_normal((1, 2, 128)) * 0.5).astype(np.float32)
    st = make_state(w.B, w.H, w.dk, w.dv, S=w.S0, xprev=w.xprev0)
    say("[scan] fused additive znorm, carried S0 and z0, in place")
    o, st2 = gpu_scan(w, S_in=st, S_out=st)
    o_ref, S_ref, z_ref, _ = oracle_scan(w)
    S, z, h = state_np(st2)
    eo, eS, ez = orc.relerr(o, o_ref), orc.relerr(S, S_ref), orc.relerr(z, z_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e} err(z)={ez:.3e}")
    assert eo <= TOL_SPLIT and eS <= TOL_SPLIT and ez <= TOL_SPLIT
    assert np.all(h == 1)


def test_fused_znorm_two_calls():
    w = additive_elu_z(1, 2, 700, seed=62)
    say("[scan] fused additive znorm, two calls cut at 300")
    o1, st = gpu_scan(w, t_slice=slice(0, 300))
    o2, st2 = gpu_scan(w, t_slice=slice(300, None), S_in=st)
    o_ref, S_ref, z_ref, _ = oracle_scan(w)
    S, z, _ = state_np(st2)
    eo = orc.relerr(np.concatenate([o1, o2], axis=2), o_ref)
    eS, ez = orc.relerr(S, S_ref), orc.relerr(z, z_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e} err(z)={ez:.3e}")
    assert eo <= TOL_SPLIT and eS <= TOL_SPLIT and ez <= TOL_SPLIT


def test_fused_znorm_segmented():
    """Segments with the normaliser: each segment's change of z from the state pass, z
    chained by the combine, then one fused pass per segment; nonzero S0 and z0."""
    w = additive_elu_z(1, 2, 8192, seed=63, beta_kind="sigmoid")
    rng = np.random.default_rng(64)
    w.S0 = (rng.standard_normal((1, 2, 128, 128)) * 0.05).astype(np.float32)
    w.xprev0 = np.abs(rng.standard_normal((1, 2, 128)) * 0.5).astype(np.float32)
    check_scan(w, tol=TOL_SPLIT)
