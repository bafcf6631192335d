"""GPU parity of the segment-parallel scan. Few heads and long sequences leave most of
the GPU idle in the ordinary scan, so the library runs P segments of each head as
virtual heads: each segment's own state change (a local and a transition pass that form
states only, or for diagonal transitions one product), a chain of the segment maps from
the caller's state, and one pass from the true start states that forms the outputs.
These shapes all take that form (P = 8 or 16); the full-size long per-channel workload
in test_gpu_full.py does too (P = 32)."""
import numpy as np
import pytest

from linear_attention_scan_amd import fwmem as F
from linear_attention_scan_amd import workloads as wl
from oracle import fwmem_oracle as orc
from tests.gpu_helpers import TOL, check_scan, gpu_scan, oracle_scan, say, state_np, flags_of, dev_tensor, f32_tensor

pytestmark = pytest.mark.gpu


def _delta(dtype="bf16", d=128, H=1, T=8192, seed=0, **kw):
    args = dict(beta_kind="two_sigmoid", lam_kind="softplus", lam_mu=-4.0)
    args.update(kw)
    return wl.make_scan(B=1, H=H, T=T, dk=d, dv=d, dtype=dtype, seed=seed,
                        name=f"segmented {dtype} d={d} H={H} T={T}", **args)


def test_segmented_split_path_delta_bf16():
    check_scan(_delta())


def test_segmented_split_path_inner_bf16():
    check_scan(_delta(H=2, seed=1, rule=wl.RULE_INNER))


def test_segmented_general_path_per_channel():
    check_scan(_delta(H=2, seed=2, beta_kind="sigmoid", lam_mu=-5.0, per_channel=True))


def test_segmented_general_path_additive_elu1():
    check_scan(wl.make_scan(B=1, H=1, T=8192, dk=128, dv=128, rule=wl.RULE_ADDITIVE, phi=wl.PHI_ELU1,
                            normalise_qk=False, beta_kind="one", lam_kind="gamma", seed=3,
                            name="segmented additive elu1"))


def test_segmented_fp32():
    check_scan(_delta(dtype="f32", d=64, seed=4))


def test_segmented_mixed_dims_and_qk_norm():
    w = wl.make_scan(B=1, H=1, T=8192, dk=64, dv=128, beta_kind="two_sigmoid", lam_kind="softplus",
                     normalise_qk=False, qk_norm="rms", seed=5, name="segmented 64x128 qk rms")
    check_scan(w)


def test_segmented_nonzero_state_in_place():
    """A nonzero initial state with a carried key, updated in place (S_in == S_out)."""
    w = _delta(H=2, seed=6)
    rng = np.random.default_rng(6)
    S0 = (rng.standard_normal((1, 2, 128, 128)) * 0.05).astype(np.float32)
    x0 = wl.round_to_bf16((rng.standard_normal((1, 2, 128)) * 0.09).astype(np.float32))
    h0 = np.array([[1, 0]], dtype=np.int32)
    from tests.gpu_helpers import make_state
    st = make_state(1, 2, 128, 128, S=S0, xprev=x0, has=h0)
    say("[segmented] nonzero S0, carried key, in place")
    o, st2 = gpu_scan(w, S_in=st, S_out=st)
    o_ref, S_ref, x_ref, _ = oracle_scan(w, S0=S0, xprev0=x0, has0=h0)
    S, x, h = state_np(st2)
    eo, eS = orc.relerr(o, o_ref), orc.relerr(S, S_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e}")
    assert eo <= TOL["bf16"] and eS <= TOL["bf16"]
    np.testing.assert_array_equal(x, x_ref.astype(np.float32).astype(np.float64))
    assert np.all(h == 1)


@pytest.mark.parametrize("case", ["per_channel_bf16", "f32"])
def test_segmented_general_path_nonzero_state(case):
    """The general pair from a nonzero initial state with a carried key: the local pass
    runs every segment from zero, so the combine chains the caller's state through
    segment 0's transition (S_start(1) = A_0 S_0 + B_0)."""
    if case == "f32":
        w, d = _delta(H=2, dtype="f32", d=64, seed=8), 64
    else:
        w, d = _delta(H=2, seed=9, beta_kind="sigmoid", lam_mu=-5.0, per_channel=True), 128
    rng = np.random.default_rng(10)
    S0 = (rng.standard_normal((1, 2, d, d)) * 0.05).astype(np.float32)
    x0 = wl.round_to_bf16((rng.standard_normal((1, 2, d)) * 0.09).astype(np.float32))
    h0 = np.array([[1, 1]], dtype=np.int32)
    from tests.gpu_helpers import make_state
    st = make_state(1, 2, d, d, S=S0, xprev=x0, has=h0)
    say(f"[segmented] general pair {case}, nonzero S0, carried key")
    o, st2 = gpu_scan(w, S_in=st)
    o_ref, S_ref, _, _ = oracle_scan(w, S0=S0, xprev0=x0, has0=h0)
    S, _, _ = state_np(st2)
    eo, eS = orc.relerr(o, o_ref), orc.relerr(S, S_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e}")
    tol = TOL["f32" if case == "f32" else "bf16"]
    assert eo <= tol and eS <= tol


@pytest.mark.parametrize("rule", [wl.RULE_DELTA, wl.RULE_ADDITIVE])
def test_segmented_propagate_is_repeatable_after_one_prep(rule):
    """prep once, then propagate twice: the propagate phase does not change its inputs, so
    both runs give the same bits (and match the oracle). The additive rule takes the
    diagonal form."""
    import torch
    w = _delta(H=2, seed=7) if rule == wl.RULE_DELTA else _delta(H=2, seed=7, rule=rule, lam_kind="gamma")
    q, k, v = (dev_tensor(a, "bf16") for a in (w.q, w.k, w.v))
    beta, lam = f32_tensor(w.beta), f32_tensor(w.lam)
    shp = F.shape(1, 2, w.T, 128, 128, F.BF16)
    md = F.mode(rule, 0, w.eps, 0)
    n = F.workspace_bytes(shp, md)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    outs = []
    st = F.State(1, 2, 128, 128)
    out0 = torch.empty((1, 2, w.T, 128), dtype=torch.float32, device="cuda")
    assert F.scan_fwd_raw(shp, q, k, v, beta, lam, md, None, out0, st.buf, ws, n, entry=F.PHASE_PREP) == F.OK
    for _ in range(2):
        out = torch.empty((1, 2, w.T, 128), dtype=torch.float32, device="cuda")
        assert F.scan_fwd_raw(shp, q, k, v, beta, lam, md, None, out, st.buf, ws, n,
                              entry=F.PHASE_PROPAGATE) == F.OK
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    o_ref, _, _, _ = oracle_scan(w)
    eo = orc.relerr(outs[0].astype(np.float64), o_ref)
    say(f"[segmented] repeat: err(o)={eo:.3e}")
    assert eo <= TOL["bf16"]


# ---- diagonal transitions: the additive rule with a scalar decay composes segments by a
# scalar (the product of the retentions), so there is no transition pass; the segments'
# own states come from one product each, and one pass from the chained start states
# forms the outputs.

def test_diagonal_segments_elu1_eight_heads():
    """Eight heads of 4096 tokens (8 segments each), C3's distributions."""
    check_scan(wl.make_scan(B=1, H=8, T=4096, dk=128, dv=128, rule=wl.RULE_ADDITIVE, phi=wl.PHI_ELU1,
                            normalise_qk=False, beta_kind="one", lam_kind="gamma", seed=11,
                            name="diagonal segments elu1 H=8"))


def test_diagonal_segments_split_pair_qk_norm_and_gate_preactivations():
    """Split pair (bf16 identity); the retention and write scale arrive as
    pre-activations (the decay kernel activates them), q and k are L2-normalised by the
    scan (the segment-state product rescales the keys)."""
    w = wl.make_scan(B=1, H=2, T=8192, dk=128, dv=128, rule=wl.RULE_ADDITIVE, normalise_qk=False,
                     qk_norm="l2", beta_kind="sigmoid", lam_kind="gamma", seed=12,
                     name="diagonal segments split qk-l2 gates-pre")
    w.gates_pre = True
    check_scan(w)


def test_diagonal_segments_no_decay_f32():
    """No retention (gamma = 1), float32, d_k = 64."""
    check_scan(wl.make_scan(B=1, H=1, T=8192, dk=64, dv=128, dtype="f32", rule=wl.RULE_ADDITIVE,
                            phi=wl.PHI_ELU1, normalise_qk=False, beta_kind="sigmoid", lam_kind="none",
                            seed=13, name="diagonal segments f32 no decay"))


def test_diagonal_segments_nonzero_state_in_place():
    w = wl.make_scan(B=1, H=2, T=8192, dk=128, dv=128, rule=wl.RULE_ADDITIVE, phi=wl.PHI_ELU1,
                     normalise_qk=False, beta_kind="one", lam_kind="gamma", gamma_mu=5.0, seed=14,
                     name="diagonal segments in place")
    rng = np.random.default_rng(14)
    S0 = (rng.standard_normal((1, 2, 128, 128)) * 0.5).astype(np.float32)
    from tests.gpu_helpers import make_state
    st = make_state(1, 2, 128, 128, S=S0)
    say("[segmented diagonal] nonzero S0, in place, slow decay (gamma ~ sigmoid(N(5, 0.5)))")
    o, st2 = gpu_scan(w, S_in=st, S_out=st)
    o_ref, S_ref, x_ref, _ = oracle_scan(w, S0=S0)
    S, x, h = state_np(st2)
    eo, eS = orc.relerr(o, o_ref), orc.relerr(S, S_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e}")
    assert eo <= TOL["bf16"] and eS <= TOL["bf16"]
    np.testing.assert_allclose(x, x_ref, rtol=4e-6, atol=1e-30)
    assert np.all(h == 1)
