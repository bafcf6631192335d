"""GPU parity of the gate activations in the load stage (FWMEM_BETA_SIGMOID,
FWMEM_BETA_SIGMOID2, FWMEM_LAMBDA_PREACT): the library receives the pre-activations
the workloads draw (beta = sigmoid(z) or 2 sigmoid(z); the ridge softplus(z); the
additive retention sigmoid(z)) and the oracle applies the same activations in fp64."""
import dataclasses

import numpy as np
import pytest

from linear_attention_scan_amd import fwmem as F
from linear_attention_scan_amd import workloads as wl
from oracle import fwmem_oracle as orc
from tests.gpu_helpers import check_scan, say

pytestmark = pytest.mark.gpu


def _pre(w):
    return dataclasses.replace(w, gates_pre=True, name=w.name + " (pre-activated gates)")


@pytest.mark.parametrize("rule", [wl.RULE_DELTA, wl.RULE_INNER])
def test_gates_split_shifted_rules(rule):
    check_scan(_pre(wl.make_scan(B=2, H=3, T=300, dk=128, dv=128, rule=rule, beta_kind="two_sigmoid",
                                 lam_kind="softplus", seed=40 + rule, name=f"rule {rule}")))


def test_gates_split_additive_retention():
    check_scan(_pre(wl.make_scan(B=2, H=2, T=300, dk=128, dv=128, rule=wl.RULE_ADDITIVE, normalise_qk=False,
                                 beta_kind="sigmoid", lam_kind="gamma", seed=43, name="additive identity")))


def test_gates_general_per_channel():
    check_scan(_pre(wl.delta_long_pc(seed=1, B=1, H=2, T=300)))


def test_gates_general_additive_elu1_per_channel():
    check_scan(_pre(wl.make_scan(B=1, H=2, T=260, dk=128, dv=128, rule=wl.RULE_ADDITIVE, phi=wl.PHI_ELU1,
                                 normalise_qk=False, beta_kind="sigmoid", lam_kind="gamma", per_channel=True,
                                 seed=44, name="additive elu1 pc")))


def test_gates_fp32_inner():
    check_scan(_pre(wl.make_scan(B=1, H=2, T=200, dk=64, dv=64, dtype="f32", rule=wl.RULE_INNER,
                                 beta_kind="sigmoid", lam_kind="softplus", lam_mu=-3.0, seed=45, name="inner f32")))


def test_gates_segmented_per_channel():
    check_scan(_pre(wl.make_scan(B=1, H=1, T=8192, dk=128, dv=128, beta_kind="sigmoid", lam_kind="softplus",
                                 lam_mu=-5.0, per_channel=True, seed=46, name="segmented pc")))


@pytest.mark.parametrize("rule,pc", [(wl.RULE_DELTA, False), (wl.RULE_DELTA, True), (wl.RULE_INNER, True),
                                     (wl.RULE_ADDITIVE, False)])
def test_gates_decode(rule, pc):
    import torch
    B, H, d, steps = 3, 4, 128, 6
    rng = np.random.default_rng(50 + rule + 3 * pc)
    S0 = (rng.standard_normal((B, H, d, d)) * 0.05).astype(np.float32)
    st = F.State(B, H, d, d)
    st.S.copy_(torch.from_numpy(S0))
    S_ref, x_ref, h_ref = S0.astype(np.float64), None, None
    flags = F.BETA_SIGMOID2 | F.LAMBDA_PREACT | (F.LAMBDA_PER_CHANNEL if pc else 0)
    outs, refs = [], []
    for s in range(steps):
        q = wl.round_to_bf16(rng.standard_normal((B, H, d)).astype(np.float32) / np.sqrt(d))
        k = wl.round_to_bf16(rng.standard_normal((B, H, d)).astype(np.float32) / np.sqrt(d))
        v = wl.round_to_bf16(rng.standard_normal((B, H, d)).astype(np.float32))
        zb = rng.standard_normal((B, H)).astype(np.float32)
        zl = (rng.standard_normal((B, H, d) if pc else (B, H)) + (3.0 if rule == wl.RULE_ADDITIVE else -4.0)).astype(np.float32)
        bt = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()
        o, _ = F.step(bt(q), bt(k), bt(v), torch.from_numpy(zb).cuda(), torch.from_numpy(zl).cuda(), rule=rule,
                      flags=flags, eps=1e-6, S_in=st, S_out=st)
        outs.append(o.cpu().numpy().astype(np.float64))
        o_ref, S_ref, x_ref, h_ref = orc.step(q, k, v, zb, zl, rule=rule, eps=1e-6, per_channel=pc, S0=S_ref,
                                              xprev0=x_ref, has0=h_ref, beta_act="sigmoid2", lam_act=True)
        refs.append(o_ref)
    torch.cuda.synchronize()
    eo = orc.relerr(np.stack(outs), np.stack(refs))
    eS = orc.relerr(st.S.cpu().numpy(), S_ref)
    say(f"[gates step] rule={rule} pc={pc}: err(o)={eo:.3e} err(S)={eS:.3e}")
    assert eo <= 1e-4 and eS <= 1e-4
