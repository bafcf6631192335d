"""GPU parity of fwmem_scan_fwd against the fp64 oracle: small and edge cases that span
several 64-token chunks with a ragged tail. Tolerances: max|x - ref|/rms(ref) <= 1e-4
(fp32 inputs) and <= 2e-2 (bf16 inputs), on the outputs o and on the final state S."""
import numpy as np
import pytest

from linear_attention_scan_amd import fwmem as F
from linear_attention_scan_amd import workloads as wl
from oracle import fwmem_oracle as orc
from tests.gpu_helpers import (check_scan, gpu_scan, make_state, oracle_scan, say, state_np, TOL)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_delta_f32_small_config(seed):
    check_scan(wl.delta_f32_small(seed=seed), label=f"delta_f32_small seed={seed}")


@pytest.mark.parametrize("seed", [0, 1])
def test_delta_bf16_ragged(seed):
    check_scan(wl.delta_bf16(seed=seed, B=2, H=3, T=300), label=f"delta_bf16 T=300 seed={seed}")


def test_delta_f32_ragged_dk128():
    w = wl.make_scan(B=2, H=2, T=200, dk=128, dv=128, dtype="f32", beta_kind="two_sigmoid",
                     lam_kind="softplus", seed=5, name="delta_f32_d128")
    check_scan(w)


def test_additive_bf16_ragged():
    check_scan(wl.additive_bf16(seed=0, B=2, H=2, T=300), label="additive_bf16 T=300")


def test_additive_f32_with_beta():
    w = wl.make_scan(B=1, H=3, T=150, dk=64, dv=64, dtype="f32", rule=wl.RULE_ADDITIVE,
                     phi=wl.PHI_ELU1, normalise_qk=False, beta_kind="sigmoid", lam_kind="gamma",
                     seed=3, name="additive_f32_beta")
    check_scan(w)


def test_delta_per_channel_bf16():
    check_scan(wl.delta_long_pc(seed=0, B=1, H=2, T=300), label="delta_pc T=300")


def test_delta_per_channel_f32():
    w = wl.make_scan(B=1, H=2, T=200, dk=64, dv=64, dtype="f32", beta_kind="sigmoid",
                     lam_kind="softplus", lam_mu=-3.0, per_channel=True, seed=4, name="delta_pc_f32")
    check_scan(w)


def test_additive_per_channel():
    w = wl.make_scan(B=1, H=2, T=260, dk=128, dv=128, dtype="bf16", rule=wl.RULE_ADDITIVE,
                     phi=wl.PHI_ELU1, normalise_qk=False, beta_kind="one", lam_kind="gamma",
                     per_channel=True, seed=6, name="additive_pc")
    check_scan(w)


def test_delta_elu1_feature_map():
    w = wl.make_scan(B=1, H=2, T=190, dk=128, dv=128, dtype="bf16", phi=wl.PHI_ELU1,
                     beta_kind="sigmoid", lam_kind="softplus", seed=7, name="delta_elu1")
    check_scan(w)


@pytest.mark.parametrize("T", [1, 2, 5, 63, 64, 65, 128, 129])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_short_sequences(T, dtype):
    d = 128 if dtype == "bf16" else 64
    w = wl.make_scan(B=1, H=2, T=T, dk=d, dv=d, dtype=dtype, beta_kind="two_sigmoid",
                     lam_kind="softplus", seed=T, name=f"short T={T}")
    check_scan(w)


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("rule", [wl.RULE_DELTA, wl.RULE_ADDITIVE])
def test_mixed_head_dims(dk, dv, rule):
    if rule == wl.RULE_DELTA:
        w = wl.make_scan(B=2, H=2, T=170, dk=dk, dv=dv, beta_kind="two_sigmoid",
                         lam_kind="softplus", seed=dk + dv, name=f"delta {dk}x{dv}")
    else:
        w = wl.make_scan(B=2, H=2, T=170, dk=dk, dv=dv, rule=rule, phi=wl.PHI_ELU1,
                         normalise_qk=False, beta_kind="one", lam_kind="gamma", seed=dk + dv,
                         name=f"additive {dk}x{dv}")
    check_scan(w)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
@pytest.mark.parametrize("beta_kind", ["one", "sigmoid"])
def test_additive_identity_bf16(dk, dv, beta_kind):
    """The additive rule with phi = identity on bf16 inputs: the split-operand kernels
    without the triangular solve. Ragged T spans several chunks and a tail; the decayed
    retention and an optional write scale come from the same draws as the additive
    workload."""
    w = wl.make_scan(B=2, H=3, T=333, dk=dk, dv=dv, rule=wl.RULE_ADDITIVE,
                     normalise_qk=False, beta_kind=beta_kind, lam_kind="gamma",
                     seed=7 * dk + dv, name=f"additive identity {dk}x{dv} beta={beta_kind}")
    check_scan(w)


def test_nonzero_initial_state_and_carried_key():
    w = wl.delta_bf16(seed=3, B=2, H=2, T=150)
    rng = np.random.default_rng(9)
    w.S0 = rng.standard_normal((2, 2, 128, 128)).astype(np.float32) * 0.05
    w.xprev0 = wl.round_to_bf16(rng.standard_normal((2, 2, 128)).astype(np.float32) * 0.09)
    w.has0 = np.array([[1, 0], [0, 1]], dtype=np.int32)
    say("[scan] nonzero S0 with carried keys")
    o, st = gpu_scan(w)
    o_ref, S_ref, _, _ = oracle_scan(w, xprev0=w.xprev0, has0=w.has0)
    S, _, _ = state_np(st)
    assert orc.relerr(o, o_ref) <= TOL["bf16"] and orc.relerr(S, S_ref) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_split_scan_carries_state(dtype):
    """scan(1..T1) then scan(T1+1..T) with the state carried equals one scan; the
    second call updates its state in place (S_in == S_out)."""
    d = 128 if dtype == "bf16" else 64
    w = wl.make_scan(B=2, H=2, T=330, dk=d, dv=d, dtype=dtype, beta_kind="two_sigmoid",
                     lam_kind="softplus", seed=11, name="split")
    T1 = 137
    say(f"[scan] split at {T1} ({dtype})")
    o1, st = gpu_scan(w, t_slice=slice(0, T1))
    o2, st2 = gpu_scan(w, t_slice=slice(T1, None), S_in=st, S_out=st)
    assert st2 is st
    o_ref, S_ref, _, _ = oracle_scan(w)
    o = np.concatenate([o1, o2], axis=2)
    S, _, _ = state_np(st)
    assert orc.relerr(o, o_ref) <= TOL[dtype] and orc.relerr(S, S_ref) <= TOL[dtype]


def test_scan_then_decode_continues_sequence():
    import torch
    w = wl.make_scan(B=2, H=3, T=133, dk=128, dv=128, beta_kind="two_sigmoid",
                     lam_kind="softplus", seed=12, name="scan+step")
    T1 = 130
    say("[scan] scan 130 tokens then 3 decode steps")
    o1, st = gpu_scan(w, t_slice=slice(0, T1))
    outs = []
    for t in range(T1, w.T):
        q = torch.from_numpy(w.q[:, :, t]).to(torch.bfloat16).cuda()
        k = torch.from_numpy(w.k[:, :, t]).to(torch.bfloat16).cuda()
        v = torch.from_numpy(w.v[:, :, t]).to(torch.bfloat16).cuda()
        beta = torch.from_numpy(np.ascontiguousarray(w.beta[:, :, t])).cuda()
        lam = torch.from_numpy(np.ascontiguousarray(w.lam[:, :, t])).cuda()
        o, _ = F.step(q, k, v, beta, lam, eps=w.eps, S_in=st, S_out=st)
        outs.append(o.float().cpu().numpy())
    torch.cuda.synchronize()
    o_ref, S_ref, _, _ = oracle_scan(w)
    o = np.concatenate([o1, np.stack(outs, axis=2)], axis=2)
    S, _, _ = state_np(st)
    assert orc.relerr(o, o_ref) <= TOL["bf16"] and orc.relerr(S, S_ref) <= TOL["bf16"]


def test_zero_beta_keeps_state():
    w = wl.make_scan(B=1, H=2, T=100, dk=128, dv=128, beta_kind=0.0, lam_kind="softplus",
                     s0_std=0.1, seed=13, name="beta0")
    check_scan(w)
    o, st = gpu_scan(w)
    S, _, _ = state_np(st)
    np.testing.assert_array_equal(S, w.S0.astype(np.float64))


def test_large_magnitudes_use_the_fp16_range_safely():
    """Values far outside fp16's range (|v| ~ 1e5, |q|,|k| ~ 1e3) go through the
    power-of-two operand scaling without overflow."""
    w = wl.make_scan(B=1, H=2, T=200, dk=128, dv=128, rule=wl.RULE_ADDITIVE, normalise_qk=False,
                     beta_kind="one", lam_kind="gamma", seed=14, name="large")
    w.q = wl.round_to_bf16(w.q * 1e3)
    w.k = wl.round_to_bf16(w.k * 1e3)
    w.v = wl.round_to_bf16(w.v * 1e5)
    check_scan(w)
    d = wl.delta_bf16(seed=15, B=1, H=2, T=200)
    d.v = wl.round_to_bf16(d.v * 1e5)
    check_scan(d, label="delta large v")
    s = wl.delta_bf16(seed=16, B=1, H=2, T=200)
    s.q = wl.round_to_bf16(s.q * 1e-6)
    s.k = wl.round_to_bf16(s.k * 1e-3)
    s.lam = (s.lam * 1e-6).astype(np.float32)
    check_scan(s, label="delta tiny keys")


def test_zero_length_copies_state():
    import torch
    w = wl.make_scan(B=2, H=2, T=0, dk=128, dv=128, s0_std=1.0, seed=17)
    st_in = make_state(2, 2, 128, 128, S=w.S0, xprev=np.ones((2, 2, 128), np.float32),
                       has=np.ones((2, 2), np.int32))
    st_out = F.State(2, 2, 128, 128)
    q = torch.zeros((2, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    out, _ = F.scan_fwd(q, q, q, None, None, S_in=st_in, S_out=st_out)
    torch.cuda.synchronize()
    assert torch.equal(st_in.buf, st_out.buf)
    st_zero = F.State(2, 2, 128, 128)
    st_zero.buf.fill_(7.0)
    F.scan_fwd(q, q, q, None, None, S_in=None, S_out=st_zero)
    torch.cuda.synchronize()
    # the padding after has_prev is not part of the state and is left alone
    for view in (st_zero.S, st_zero.x_prev, st_zero.has_prev):
        assert float(view.abs().max()) == 0.0


def test_out_bf16_is_the_rounded_fp32_output():
    import torch
    w = wl.delta_bf16(seed=18, B=1, H=2, T=140)
    o32, _ = gpu_scan(w)
    o16, _ = gpu_scan(w, extra_flags=F.OUT_BF16)
    want = torch.from_numpy(o32.astype(np.float32)).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(o16.astype(np.float32), want)


def test_repeated_runs_are_bit_identical():
    w = wl.delta_long_pc(seed=19, B=1, H=2, T=200)
    a, sa = gpu_scan(w)
    b, sb = gpu_scan(w)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(state_np(sa)[0], state_np(sb)[0])
