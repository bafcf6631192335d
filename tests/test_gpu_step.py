"""GPU parity of fwmem_step (one-token decode) against the fp64 oracle."""
import numpy as np
import pytest

from linear_attention_scan_amd import fwmem as F
from linear_attention_scan_amd import workloads as wl
from oracle import fwmem_oracle as orc
from tests.gpu_helpers import TOL, make_state, say

pytestmark = pytest.mark.gpu


def _t(x, bf16=True):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    return (t.to(torch.bfloat16) if bf16 else t).cuda()


@pytest.mark.parametrize("rule,pc,dtype,dk,dv", [
    (wl.RULE_DELTA, False, "bf16", 128, 128),
    (wl.RULE_DELTA, True, "bf16", 128, 128),
    (wl.RULE_DELTA, False, "f32", 64, 64),
    (wl.RULE_DELTA, False, "bf16", 64, 128),
    (wl.RULE_DELTA, True, "f32", 128, 64),
    (wl.RULE_ADDITIVE, False, "bf16", 128, 128),
    (wl.RULE_ADDITIVE, True, "f32", 64, 128),
    (wl.RULE_INNER, False, "bf16", 128, 128),
    (wl.RULE_INNER, True, "bf16", 128, 64),
    (wl.RULE_INNER, False, "f32", 64, 64),
])
def test_step_sequence_matches_oracle(rule, pc, dtype, dk, dv):
    """Several steps from a random S0 with no previous key: step 1 reads only, later
    steps write; in place (S_in == S_out) after the first step."""
    import torch
    B, H, steps = 3, 5, 6
    rng = np.random.default_rng(dk + dv + 7 * pc + 11 * rule)
    S0 = (rng.standard_normal((B, H, dk, dv)) * 0.05).astype(np.float32)
    say(f"[step] rule={rule} pc={pc} {dtype} dk={dk} dv={dv}")
    st_in = make_state(B, H, dk, dv, S=S0)
    st = F.State(B, H, dk, dv)
    S_ref, x_ref, h_ref = S0.astype(np.float64), None, None
    flags = (F.LAMBDA_PER_CHANNEL if pc else 0) | (F.PHI_ELU1 if rule == wl.RULE_ADDITIVE else 0)
    phi = "elu1" if rule == wl.RULE_ADDITIVE else "identity"
    outs, refs = [], []
    for s in range(steps):
        q = rng.standard_normal((B, H, dk)).astype(np.float32)
        k = rng.standard_normal((B, H, dk)).astype(np.float32)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((B, H, dv)).astype(np.float32)
        if dtype == "bf16":
            q, k, v = wl.round_to_bf16(q), wl.round_to_bf16(k), wl.round_to_bf16(v)
        beta = rng.uniform(0.1, 1.9, size=(B, H)).astype(np.float32)
        if rule != wl.RULE_ADDITIVE:
            lam = rng.uniform(0, 0.2, size=(B, H, dk) if pc else (B, H)).astype(np.float32)
        else:
            lam = rng.uniform(0.8, 1.0, size=(B, H, dk) if pc else (B, H)).astype(np.float32)
        o, _ = F.step(_t(q, dtype == "bf16"), _t(k, dtype == "bf16"), _t(v, dtype == "bf16"),
                      _t(beta, False), _t(lam, False), rule=rule, flags=flags, eps=1e-6,
                      S_in=st_in if s == 0 else st, S_out=st)
        outs.append(o.cpu().numpy().astype(np.float64))
        o_ref, S_ref, x_ref, h_ref = orc.step(q, k, v, beta, lam, rule=rule, phi_kind=phi, eps=1e-6,
                                              per_channel=pc, S0=S_ref, xprev0=x_ref, has0=h_ref)
        refs.append(o_ref)
    torch.cuda.synchronize()
    eo = orc.relerr(np.stack(outs), np.stack(refs))
    eS = orc.relerr(st.S.cpu().numpy(), S_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e}")
    # the decode kernel is plain fp32 arithmetic for both input types
    assert eo <= TOL["f32"] and eS <= TOL["f32"]
    assert np.all(st.has_prev.cpu().numpy() == 1)


def test_step_first_token_reads_only():
    import torch
    B, H, d = 2, 3, 128
    rng = np.random.default_rng(1)
    S0 = rng.standard_normal((B, H, d, d)).astype(np.float32)
    st_in = make_state(B, H, d, d, S=S0)
    q = wl.round_to_bf16(rng.standard_normal((B, H, d)).astype(np.float32))
    kv = wl.round_to_bf16(rng.standard_normal((B, H, d)).astype(np.float32))
    beta = np.full((B, H), 1.5, np.float32)
    lam = np.full((B, H), 3.0, np.float32)
    st = F.State(B, H, d, d)
    o, _ = F.step(_t(q), _t(kv), _t(kv), _t(beta, False), _t(lam, False), S_in=st_in, S_out=st)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(st.S.cpu().numpy(), S0)
    np.testing.assert_allclose(o.cpu().numpy(), np.einsum("bhij,bhi->bhj", S0, q), rtol=1e-5, atol=1e-4)
    np.testing.assert_array_equal(st.x_prev.cpu().numpy(), kv)


def test_step_out_bf16_is_rounded_fp32():
    import torch
    B, H, d = 4, 4, 128
    rng = np.random.default_rng(2)
    S0 = rng.standard_normal((B, H, d, d)).astype(np.float32)
    q = wl.round_to_bf16(rng.standard_normal((B, H, d)).astype(np.float32))
    beta = np.full((B, H), 0.5, np.float32)
    a = F.step(_t(q), _t(q), _t(q), _t(beta, False), None, S_in=make_state(B, H, d, d, S=S0))[0]
    b = F.step(_t(q), _t(q), _t(q), _t(beta, False), None, S_in=make_state(B, H, d, d, S=S0),
               flags=F.OUT_BF16)[0]
    torch.cuda.synchronize()
    assert torch.equal(a.to(torch.bfloat16), b)
