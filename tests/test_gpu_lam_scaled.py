"""GPU parity of the scale-coupled ridge (FWMEM_LAMBDA_SCALED: lambda is a base ridge
times the energy of the written key) against the fp64 oracle, on both kernel pairs, with
QK normalisation, in the segmented form and in decode. The keys are left unnormalised
(|x|^2 near d_k) so that the coupling changes the ridge by two orders of magnitude."""
import numpy as np
import pytest

from linear_attention_scan_amd import fwmem as F
from linear_attention_scan_amd import workloads as wl
from oracle import fwmem_oracle as orc
from tests.gpu_helpers import TOL, check_scan, make_state, say, state_np

pytestmark = pytest.mark.gpu


def _scaled(B=2, H=3, T=1000, dk=128, dv=128, dtype="bf16", rule=wl.RULE_DELTA, seed=0, **kw):
    args = dict(beta_kind="two_sigmoid", lam_kind="softplus", lam_mu=-4.0, normalise_qk=False)
    args.update(kw)
    return wl.make_scan(B=B, H=H, T=T, dk=dk, dv=dv, dtype=dtype, rule=rule, seed=seed,
                        lam_scaled=True, name=f"scaled ridge rule={rule} {dtype} {dk}x{dv} T={T}",
                        **args)


@pytest.mark.parametrize("rule,d,T", [(wl.RULE_DELTA, 128, 1000), (wl.RULE_INNER, 64, 333)])
def test_scaled_ridge_split_pair(rule, d, T):
    check_scan(_scaled(rule=rule, dk=d, dv=d, T=T, seed=d + rule))


def test_scaled_ridge_with_qk_rmsnorm():
    """After RMSNorm every key has energy d_k, so the ridge is d_k times the base."""
    check_scan(_scaled(T=700, seed=1, qk_norm="rms"))


@pytest.mark.parametrize("rule", [wl.RULE_DELTA, wl.RULE_INNER])
def test_scaled_ridge_general_pair_f32(rule):
    check_scan(_scaled(B=1, H=2, T=700, dk=64, dv=128, dtype="f32", rule=rule, seed=2))


def test_scaled_ridge_general_pair_elu1():
    check_scan(_scaled(B=1, H=2, T=640, phi=wl.PHI_ELU1, seed=3))


def test_scaled_ridge_segmented():
    check_scan(_scaled(B=1, H=1, T=8192, seed=4), label="scaled ridge segmented")


@pytest.mark.parametrize("rule,pc,dtype,dk,dv", [
    (wl.RULE_DELTA, False, "bf16", 128, 128),
    (wl.RULE_DELTA, True, "f32", 64, 128),
    (wl.RULE_INNER, False, "bf16", 128, 64),
    (wl.RULE_INNER, True, "bf16", 64, 64),
])
def test_scaled_ridge_decode_sequence(rule, pc, dtype, dk, dv):
    """Decode steps from a random S0 with unnormalised keys, in place after the first."""
    import torch
    B, H, steps = 3, 4, 6
    rng = np.random.default_rng(dk + dv + 7 * pc + 11 * rule)
    S0 = (rng.standard_normal((B, H, dk, dv)) * 0.05).astype(np.float32)
    say(f"[scaled ridge step] rule={rule} pc={pc} {dtype} dk={dk} dv={dv}")
    st_in = make_state(B, H, dk, dv, S=S0)
    st = F.State(B, H, dk, dv)
    S_ref, x_ref, h_ref = S0.astype(np.float64), None, None
    flags = F.LAMBDA_SCALED | (F.LAMBDA_PER_CHANNEL if pc else 0)
    bf = dtype == "bf16"

    def t(x, b):
        y = torch.from_numpy(np.ascontiguousarray(x))
        return (y.to(torch.bfloat16) if b else y).cuda()

    outs, refs = [], []
    for s in range(steps):
        q, k = (rng.standard_normal((B, H, dk)).astype(np.float32) for _ in range(2))
        v = rng.standard_normal((B, H, dv)).astype(np.float32)
        if bf:
            q, k, v = wl.round_to_bf16(q), wl.round_to_bf16(k), wl.round_to_bf16(v)
        beta = rng.uniform(0.1, 1.9, size=(B, H)).astype(np.float32)
        lam = rng.uniform(0.0, 0.05, size=(B, H, dk) if pc else (B, H)).astype(np.float32)
        o, _ = F.step(t(q, bf), t(k, bf), t(v, bf), t(beta, False), t(lam, False), rule=rule,
                      flags=flags, eps=1e-6, S_in=st_in if s == 0 else st, S_out=st)
        outs.append(o.cpu().numpy().astype(np.float64))
        o_ref, S_ref, x_ref, h_ref = orc.step(q, k, v, beta, lam, rule=rule, eps=1e-6,
                                              per_channel=pc, S0=S_ref, xprev0=x_ref, has0=h_ref,
                                              lam_scaled=True)
        refs.append(o_ref)
    torch.cuda.synchronize()
    S, _, h = state_np(st)
    eo, eS = orc.relerr(np.stack(outs), np.stack(refs)), orc.relerr(S, S_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e}")
    assert eo <= TOL["f32"] and eS <= TOL["f32"]
    assert np.all(h == 1)
