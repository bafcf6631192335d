"""GPU parity of the fused query/key normalisation (FWMEM_QK_L2NORM: unit length,
FWMEM_QK_RMSNORM: RMS 1 with unit gain; "Fast Weight Attention for Continual Learning"
reading notes, section 4.5) against the fp64 oracle on raw, unnormalised q and k.
The library folds the per-token rescale factors into the prep kernels' masks and row
factors, so the raw bf16 rows stay exact MFMA operands. Tolerances as elsewhere:
max|x - ref|/rms(ref) <= 1e-4 (fp32 inputs) and <= 2e-2 (bf16 inputs)."""
import numpy as np
import pytest

from linear_attention_scan_amd import fwmem as F
from linear_attention_scan_amd import workloads as wl
from oracle import fwmem_oracle as orc
from tests.gpu_helpers import TOL, check_scan, gpu_scan, oracle_scan, say, state_np

pytestmark = pytest.mark.gpu

RULES = {"delta": wl.RULE_DELTA, "inner": wl.RULE_INNER, "additive": wl.RULE_ADDITIVE}


def _raw(rule, mode, B, H, T, dk, dv, dtype="bf16", seed=0, **kw):
    r = RULES[rule]
    args = dict(beta_kind="two_sigmoid", lam_kind="softplus", lam_mu=-4.0)
    if r == wl.RULE_ADDITIVE:
        args = dict(beta_kind="sigmoid", lam_kind="gamma")
    args.update(kw)
    return wl.make_scan(B=B, H=H, T=T, dk=dk, dv=dv, dtype=dtype, rule=r, normalise_qk=False,
                        qk_norm=mode, seed=seed, name=f"{rule} {mode} {dtype} {dk}x{dv} T={T}", **args)


@pytest.mark.parametrize("mode", ["l2", "rms"])
@pytest.mark.parametrize("rule", ["delta", "inner", "additive"])
def test_qknorm_split_bf16(rule, mode):
    check_scan(_raw(rule, mode, 2, 3, 300, 128, 128, seed=len(rule) + len(mode)))


@pytest.mark.parametrize("mode", ["l2", "rms"])
@pytest.mark.parametrize("rule", ["delta", "inner", "additive"])
def test_qknorm_general_f32(rule, mode):
    check_scan(_raw(rule, mode, 1, 2, 200, 64, 64, dtype="f32", seed=3 + len(rule)))


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
def test_qknorm_mixed_head_dims(dk, dv):
    check_scan(_raw("delta", "l2", 2, 2, 170, dk, dv, seed=dk + dv))


def test_qknorm_per_channel_bf16():
    check_scan(_raw("delta", "rms", 1, 2, 260, 128, 128, seed=9, beta_kind="sigmoid", lam_mu=-5.0,
                    per_channel=True))


def test_qknorm_wide_token_scales():
    """Per-token magnitudes of q and k spread over six decades: the normalised scan sees
    none of it (the oracle normalises in fp64)."""
    w = _raw("delta", "l2", 1, 2, 200, 128, 128, seed=12)
    rng = np.random.default_rng(5)
    w.q = wl.round_to_bf16(w.q * (10.0 ** rng.uniform(-3, 3, (1, 2, 200, 1))).astype(np.float32))
    w.k = wl.round_to_bf16(w.k * (10.0 ** rng.uniform(-3, 3, (1, 2, 200, 1))).astype(np.float32))
    check_scan(w, label="qk l2, token scales 1e-3..1e3")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_qknorm_carries_the_raw_key_across_scans_and_steps(dtype):
    import torch
    d = 128 if dtype == "bf16" else 64
    w = _raw("delta", "rms", 2, 2, 200, d, d, dtype=dtype, seed=21)
    T1, T2 = 70, 190
    say(f"[qknorm] carry {dtype}: scan to {T1}, scan to {T2}, {w.T - T2} steps")
    o1, st = gpu_scan(w, t_slice=slice(0, T1))
    o2, _ = gpu_scan(w, t_slice=slice(T1, T2), S_in=st, S_out=st)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    steps = []
    for t in range(T2, w.T):
        cv = lambda x: torch.from_numpy(np.ascontiguousarray(x[:, :, t])).to(tdt).cuda()
        cf = lambda x: torch.from_numpy(np.ascontiguousarray(x[:, :, t])).cuda()
        o, _ = F.step(cv(w.q), cv(w.k), cv(w.v), cf(w.beta), cf(w.lam), rule=w.rule,
                      flags=F.QK_RMSNORM, eps=w.eps, S_in=st, S_out=st)
        steps.append(o.float().cpu().numpy()[:, :, None].astype(np.float64))
    torch.cuda.synchronize()
    o = np.concatenate([o1, o2] + steps, axis=2)
    o_ref, S_ref, x_ref, _ = oracle_scan(w)
    S, x, _ = state_np(st)
    eo, eS = orc.relerr(o, o_ref), orc.relerr(S, S_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e}")
    assert eo <= TOL[dtype] and eS <= TOL[dtype]
    np.testing.assert_array_equal(x, x_ref.astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("rule", ["delta", "inner", "additive"])
@pytest.mark.parametrize("mode", ["l2", "rms"])
def test_qknorm_decode_steps(rule, mode):
    import torch
    B, H, d, steps = 3, 4, 128, 6
    r = RULES[rule]
    flag = F.QK_L2NORM if mode == "l2" else F.QK_RMSNORM
    rng = np.random.default_rng(len(rule) * 7 + len(mode))
    S0 = (rng.standard_normal((B, H, d, d)) * 0.05).astype(np.float32)
    st = F.State(B, H, d, d)
    st.S.copy_(torch.from_numpy(S0))
    S_ref, x_ref, h_ref = S0.astype(np.float64), None, None
    outs, refs = [], []
    for s in range(steps):
        q = wl.round_to_bf16((rng.standard_normal((B, H, d)) * 3).astype(np.float32))
        k = wl.round_to_bf16((rng.standard_normal((B, H, d)) * 0.2).astype(np.float32))
        v = wl.round_to_bf16(rng.standard_normal((B, H, d)).astype(np.float32))
        beta = rng.uniform(0.1, 1.9, (B, H)).astype(np.float32)
        lam = (rng.uniform(0, 0.2, (B, H)) if r != wl.RULE_ADDITIVE else rng.uniform(0.8, 1.0, (B, H))).astype(np.float32)
        bt = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
        o, _ = F.step(bt(q), bt(k), bt(v), torch.from_numpy(beta).cuda(), torch.from_numpy(lam).cuda(),
                      rule=r, flags=flag, eps=1e-6, S_in=st, S_out=st)
        outs.append(o.cpu().numpy().astype(np.float64))
        o_ref, S_ref, x_ref, h_ref = orc.step(q, k, v, beta, lam, rule=r, eps=1e-6, S0=S_ref,
                                              xprev0=x_ref, has0=h_ref, qk_norm=mode)
        refs.append(o_ref)
    torch.cuda.synchronize()
    eo = orc.relerr(np.stack(outs), np.stack(refs))
    eS = orc.relerr(st.S.cpu().numpy(), S_ref)
    say(f"[qknorm step] {rule} {mode}: err(o)={eo:.3e} err(S)={eS:.3e}")
    assert eo <= 1e-4 and eS <= 1e-4
    np.testing.assert_array_equal(st.x_prev.cpu().numpy(), x_ref.astype(np.float32))


@pytest.mark.slow
def test_qknorm_full_throughput_shape():
    check_scan(wl.delta_bf16_h16_qknorm(seed=0), label="delta_bf16_h16_qknorm B=4 H=16 T=4096")


def test_qknorm_zero_rows_stay_zero():
    """Zero query and key rows (padding tokens) normalise to zero in the oracle (reading
    D16) and in the library: no division by zero, and the scan matches."""
    w = _raw("delta", "l2", 1, 2, 200, 128, 128, seed=31)
    w.q[:, :, 40:50] = 0.0
    w.k[:, :, 60:75] = 0.0
    w.k[:, :, -1] = 0.0
    check_scan(w, label="qk l2 with zero rows")
