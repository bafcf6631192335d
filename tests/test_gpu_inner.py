"""GPU parity of the inner-product rule (Falcon-1A: the shifted pair, the normalised
step and the decay of the delta rule, with the target written in place of the
residual; "Fast Weight Attention for Continual Learning" reading notes, section 4.3)
against the fp64 oracle, through the C ABI. Both kernel pairs are covered: the split
pair (bf16 inputs, identity map, scalar decay) and the general pair (fp32 inputs,
elu+1, per-channel decay). Tolerances as for the other rules: max|x - ref|/rms(ref)
<= 1e-4 (fp32 inputs) and <= 2e-2 (bf16 inputs), on o and on the final S."""
import numpy as np
import pytest

from linear_attention_scan_amd import fwmem as F
from linear_attention_scan_amd import workloads as wl
from oracle import fwmem_oracle as orc
from tests.gpu_helpers import TOL, check_scan, gpu_scan, oracle_scan, say, state_np

pytestmark = pytest.mark.gpu


def _inner(B, H, T, dk, dv, dtype="bf16", seed=0, **kw):
    args = dict(beta_kind="two_sigmoid", lam_kind="softplus", lam_mu=-4.0)
    args.update(kw)
    return wl.make_scan(B=B, H=H, T=T, dk=dk, dv=dv, dtype=dtype, rule=wl.RULE_INNER, seed=seed,
                        name=f"inner {dtype} {dk}x{dv} T={T}", **args)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_inner_f32_small_config(seed):
    check_scan(wl.inner_f32_small(seed=seed), label=f"inner_f32_small seed={seed}")


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 129, 300])
def test_inner_bf16_split_ragged(T):
    check_scan(_inner(2, 3, T, 128, 128, seed=T))


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64), (64, 64)])
def test_inner_bf16_mixed_head_dims(dk, dv):
    check_scan(_inner(2, 2, 170, dk, dv, seed=dk + 3 * dv))


def test_inner_f32_ragged_d128():
    check_scan(_inner(1, 2, 200, 128, 128, dtype="f32", seed=5))


def test_inner_per_channel_bf16():
    check_scan(_inner(1, 2, 300, 128, 128, seed=6, beta_kind="sigmoid", lam_mu=-5.0,
                      per_channel=True))


def test_inner_per_channel_f32():
    check_scan(_inner(1, 2, 200, 64, 64, dtype="f32", seed=7, beta_kind="sigmoid", lam_mu=-3.0,
                      per_channel=True))


def test_inner_elu1_feature_map():
    check_scan(_inner(1, 2, 190, 128, 128, seed=8, phi=wl.PHI_ELU1, normalise_qk=False,
                      beta_kind="sigmoid"))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_inner_split_scan_and_decode_carry_state(dtype):
    """scan(1..T1), then scan(T1+1..T2) in place, then single steps to T: the carried
    key and state cross both kinds of call boundary."""
    import torch
    d = 128 if dtype == "bf16" else 64
    w = _inner(2, 2, 200, d, d, dtype=dtype, seed=11)
    T1, T2 = 70, 190
    say(f"[inner] carry {dtype}: scan to {T1}, scan to {T2}, {w.T - T2} steps")
    o1, st = gpu_scan(w, t_slice=slice(0, T1))
    o2, _ = gpu_scan(w, t_slice=slice(T1, T2), S_in=st, S_out=st)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    steps = []
    for t in range(T2, w.T):
        cv = lambda x: torch.from_numpy(np.ascontiguousarray(x[:, :, t])).to(tdt).cuda()
        cf = lambda x: torch.from_numpy(np.ascontiguousarray(x[:, :, t])).cuda()
        o, _ = F.step(cv(w.q), cv(w.k), cv(w.v), cf(w.beta), cf(w.lam), rule=wl.RULE_INNER,
                      eps=w.eps, S_in=st, S_out=st)
        steps.append(o.float().cpu().numpy()[:, :, None].astype(np.float64))
    torch.cuda.synchronize()
    o = np.concatenate([o1, o2] + steps, axis=2)
    o_ref, S_ref, _, _ = oracle_scan(w)
    S, _, _ = state_np(st)
    eo, eS = orc.relerr(o, o_ref), orc.relerr(S, S_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e}")
    assert eo <= TOL[dtype] and eS <= TOL[dtype]


def test_inner_nonzero_initial_state_and_carried_key():
    w = _inner(2, 2, 150, 128, 128, seed=3)
    rng = np.random.default_rng(9)
    w.S0 = rng.standard_normal((2, 2, 128, 128)).astype(np.float32) * 0.05
    w.xprev0 = wl.round_to_bf16(rng.standard_normal((2, 2, 128)).astype(np.float32) * 0.09)
    w.has0 = np.array([[1, 0], [0, 1]], dtype=np.int32)
    say("[inner] nonzero S0 with carried keys")
    o, st = gpu_scan(w)
    o_ref, S_ref, _, _ = oracle_scan(w, xprev0=w.xprev0, has0=w.has0)
    S, _, _ = state_np(st)
    eo, eS = orc.relerr(o, o_ref), orc.relerr(S, S_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e}")
    assert eo <= TOL["bf16"] and eS <= TOL["bf16"]


@pytest.mark.slow
def test_inner_full_bf16():
    check_scan(wl.inner_bf16(seed=0), label="inner_bf16 B=4 H=8 T=4096")
