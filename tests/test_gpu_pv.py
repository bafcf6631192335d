"""GPU parity of the per-value-channel delta rule (Falcon-2, FWMEM_RULE_DELTA_PV: one
step size per value channel) against the fp64 oracle: scans with a ragged tail, both
input types and both key widths, QK normalisation with the scale-coupled ridge and gate
pre-activations, elu+1 features, a carried state in place across two calls, the
prep/propagate split, and decode."""
import numpy as np
import pytest

from linear_attention_scan_amd import fwmem as F
from linear_attention_scan_amd import workloads as wl
from oracle import fwmem_oracle as orc
from tests.gpu_helpers import (TOL, check_scan, dev_tensor, f32_tensor, gpu_scan, make_state,
                               oracle_scan, say, state_np)

pytestmark = pytest.mark.gpu


def _pv(B=2, H=3, T=1000, dk=128, dv=128, dtype="bf16", seed=0, **kw):
    args = dict(beta_kind="two_sigmoid", lam_kind="softplus", lam_mu=-4.0)
    args.update(kw)
    return wl.make_scan(B=B, H=H, T=T, dk=dk, dv=dv, dtype=dtype, rule=wl.RULE_DELTA_PV, seed=seed,
                        name=f"per-value-channel {dtype} {dk}x{dv} T={T}", **args)


@pytest.mark.parametrize("dtype,dk,dv,T", [
    ("bf16", 128, 128, 1000), ("bf16", 64, 128, 333), ("f32", 64, 64, 300), ("f32", 128, 64, 64),
    ("bf16", 128, 128, 1),
])
def test_pv_scan(dtype, dk, dv, T):
    check_scan(_pv(dtype=dtype, dk=dk, dv=dv, T=T, seed=dk + dv + T))


def test_pv_qk_norm_scaled_ridge_gate_preactivations():
    w = _pv(T=700, seed=1, normalise_qk=False, qk_norm="rms", lam_scaled=True)
    w.gates_pre = True
    check_scan(w)


def test_pv_elu1():
    check_scan(_pv(B=1, H=2, T=500, seed=2, phi=wl.PHI_ELU1, normalise_qk=False,
                   beta_kind="sigmoid", lam_kind="const", lam_const=0.5))


def test_pv_two_calls_in_place():
    """Nonzero S0, a scan cut at token 640 with the state updated in place between the
    calls (the carried key crosses the cut)."""
    w = _pv(B=1, H=2, T=1000, seed=3)
    rng = np.random.default_rng(3)
    S0 = (rng.standard_normal((1, 2, 128, 128)) * 0.05).astype(np.float32)
    st = make_state(1, 2, 128, 128, S=S0)
    say("[pv] two calls, in place")
    o1, _ = gpu_scan(w, t_slice=slice(0, 640), S_in=st, S_out=st)
    o2, _ = gpu_scan(w, t_slice=slice(640, None), S_in=st, S_out=st)
    o_ref, S_ref, x_ref, _ = oracle_scan(w, S0=S0)
    S, x, h = state_np(st)
    o = np.concatenate([o1, o2], axis=2)
    eo, eS = orc.relerr(o, o_ref), orc.relerr(S, S_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e}")
    assert eo <= TOL["bf16"] and eS <= TOL["bf16"]
    np.testing.assert_array_equal(x, x_ref.astype(np.float32).astype(np.float64))
    assert np.all(h == 1)


def test_pv_propagate_repeatable_after_one_prep():
    import torch
    w = _pv(B=1, H=2, T=777, seed=4)
    q, k, v = (dev_tensor(a, "bf16") for a in (w.q, w.k, w.v))
    beta, lam = f32_tensor(w.beta), f32_tensor(w.lam)
    shp = F.shape(1, 2, w.T, 128, 128, F.BF16)
    md = F.mode(wl.RULE_DELTA_PV, 0, w.eps, 0)
    n = F.workspace_bytes(shp, md)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    st = F.State(1, 2, 128, 128)
    out0 = torch.empty((1, 2, w.T, 128), dtype=torch.float32, device="cuda")
    assert F.scan_fwd_raw(shp, q, k, v, beta, lam, md, None, out0, st.buf, ws, n, entry=F.PHASE_PREP) == F.OK
    outs = []
    for _ in range(2):
        out = torch.empty((1, 2, w.T, 128), dtype=torch.float32, device="cuda")
        assert F.scan_fwd_raw(shp, q, k, v, beta, lam, md, None, out, st.buf, ws, n,
                              entry=F.PHASE_PROPAGATE) == F.OK
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0], outs[1])
    eo = orc.relerr(outs[0].astype(np.float64), oracle_scan(w)[0])
    say(f"[pv] repeat: err(o)={eo:.3e}")
    assert eo <= TOL["bf16"]


@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 64, 128), ("bf16", 128, 64)])
def test_pv_decode_sequence(dtype, dk, dv):
    import torch
    B, H, steps = 3, 4, 6
    rng = np.random.default_rng(dk + 3 * dv)
    S0 = (rng.standard_normal((B, H, dk, dv)) * 0.05).astype(np.float32)
    say(f"[pv step] {dtype} dk={dk} dv={dv}")
    st_in = make_state(B, H, dk, dv, S=S0)
    st = F.State(B, H, dk, dv)
    S_ref, x_ref, h_ref = S0.astype(np.float64), None, None
    bf = dtype == "bf16"

    def t(x, b):
        y = torch.from_numpy(np.ascontiguousarray(x))
        return (y.to(torch.bfloat16) if b else y).cuda()

    outs, refs = [], []
    for s in range(steps):
        q, k = (rng.standard_normal((B, H, dk)).astype(np.float32) for _ in range(2))
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((B, H, dv)).astype(np.float32)
        if bf:
            q, k, v = wl.round_to_bf16(q), wl.round_to_bf16(k), wl.round_to_bf16(v)
        beta = rng.uniform(0.1, 1.9, size=(B, H, dv)).astype(np.float32)
        lam = rng.uniform(0.0, 0.2, size=(B, H)).astype(np.float32)
        o, _ = F.step(t(q, bf), t(k, bf), t(v, bf), t(beta, False), t(lam, False),
                      rule=wl.RULE_DELTA_PV, eps=1e-6, S_in=st_in if s == 0 else st, S_out=st)
        outs.append(o.cpu().numpy().astype(np.float64))
        o_ref, S_ref, x_ref, h_ref = orc.step(q, k, v, beta, lam, rule=wl.RULE_DELTA_PV, eps=1e-6,
                                              S0=S_ref, xprev0=x_ref, has0=h_ref)
        refs.append(o_ref)
    torch.cuda.synchronize()
    S, _, h = state_np(st)
    eo, eS = orc.relerr(np.stack(outs), np.stack(refs)), orc.relerr(S, S_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e}")
    assert eo <= TOL["f32"] and eS <= TOL["f32"]
    assert np.all(h == 1)


@pytest.mark.parametrize("T", [63, 64, 65, 129])
def test_pv_chunk_boundaries(T):
    check_scan(_pv(B=1, H=2, T=T, seed=10 + T))


def test_pv_out_bf16_is_rounded_fp32():
    """bf16 outputs are the fp32 outputs rounded to nearest even."""
    import torch
    w = _pv(B=1, H=2, T=200, seed=20)
    o32, _ = gpu_scan(w)
    o16, _ = gpu_scan(w, extra_flags=F.OUT_BF16)
    ref = torch.from_numpy(o32.astype(np.float32)).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(o16, ref.astype(np.float64))


def test_pv_scan_then_decode():
    """A scan's final state continues in decode steps, against the oracle over the whole
    sequence."""
    import torch
    w = _pv(B=1, H=2, T=130, seed=21)
    say("[pv] scan of 127 tokens, then 3 decode steps")
    _, st = gpu_scan(w, t_slice=slice(0, 127))
    outs = []
    for t in range(127, 130):
        q, k, v = (dev_tensor(a[:, :, t], "bf16") for a in (w.q, w.k, w.v))
        o, _ = F.step(q, k, v, f32_tensor(w.beta[:, :, t]), f32_tensor(w.lam[:, :, t]),
                      rule=wl.RULE_DELTA_PV, eps=w.eps, S_in=st, S_out=st)
        outs.append(o.float().cpu().numpy())
    torch.cuda.synchronize()
    o_ref, S_ref, _, _ = oracle_scan(w)
    eo = orc.relerr(np.stack(outs, axis=2).astype(np.float64), o_ref[:, :, 127:])
    eS = orc.relerr(state_np(st)[0], S_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e}")
    assert eo <= TOL["bf16"] and eS <= TOL["bf16"]
