"""GPU parity of normalised linear attention (FWMEM_ZNORM, additive rule) against the fp64
oracle: scans on both kernel pairs (the split pair for bf16 identity features, the
general pair for elu+1 and float32), a ragged tail, a carried state updated in place, a
scan cut in two, the segmented form, an empty scan, and the one-token decode.

The features are kept positive (elu+1, or |N(0,1)| queries and keys for the identity
map) so that the normaliser is a sum of positive terms, as in the page's linear
attention; with features of either sign z . q can pass through zero and the outputs are
then not defined to any precision."""
import numpy as np
import pytest

from linear_attention_scan_amd import fwmem as F
from linear_attention_scan_amd import workloads as wl
from oracle import fwmem_oracle as orc
from tests.gpu_helpers import TOL, check_scan, gpu_scan, make_state, oracle_scan, say, state_np

pytestmark = pytest.mark.gpu


def _identity(B=2, H=3, T=1000, d=128, dtype="bf16", seed=0, **kw):
    args = dict(beta_kind="sigmoid", lam_kind="gamma", gamma_mu=3.0, gamma_sd=0.5,
                normalise_qk=True, qk_positive=True)
    args.update(kw)
    return wl.make_scan(B=B, H=H, T=T, dk=d, dv=d, dtype=dtype, rule=wl.RULE_ADDITIVE,
                        seed=seed, znorm=True, name=f"znorm identity {dtype} d={d} T={T}", **args)


def _elu1(B=1, H=3, T=1500, dk=128, dv=128, dtype="bf16", seed=0, **kw):
    args = dict(beta_kind="one", lam_kind="gamma", gamma_mu=3.0, gamma_sd=0.5, normalise_qk=False)
    args.update(kw)
    return wl.make_scan(B=B, H=H, T=T, dk=dk, dv=dv, dtype=dtype, rule=wl.RULE_ADDITIVE,
                        phi=wl.PHI_ELU1, seed=seed, znorm=True,
                        name=f"znorm elu1 {dtype} {dk}x{dv} T={T}", **args)


@pytest.mark.parametrize("d,T", [(128, 1000), (64, 333)])
def test_znorm_split_pair_identity(d, T):
    check_scan(_identity(d=d, T=T, seed=d))


def test_znorm_split_pair_qk_l2norm():
    """Raw positive q, k normalised by the scan (the QK factors reach the normaliser's
    chunk terms too)."""
    check_scan(_identity(T=700, seed=1, normalise_qk=False, qk_norm="l2"))


def test_znorm_general_pair_elu1_bf16():
    check_scan(_elu1(seed=2))


@pytest.mark.parametrize("phi", ["elu1", "identity"])
def test_znorm_general_pair_f32(phi):
    if phi == "elu1":
        w = _elu1(B=1, H=2, T=700, dk=64, dv=128, dtype="f32", seed=3)
    else:
        w = _identity(B=1, H=2, T=700, d=64, dtype="f32", seed=3)
    check_scan(w)


def test_znorm_workload_small():
    """The additive_znorm_bf16 workload's recipe at a size the oracle finishes quickly."""
    check_scan(wl.additive_znorm_bf16(seed=4, B=1, H=2, T=2048))


@pytest.mark.parametrize("pair", ["split", "general"])
def test_znorm_carried_state_in_place(pair):
    """Nonzero S0 and z0, state updated in place (S_in == S_out)."""
    w = (_identity(B=1, H=2, T=640, seed=5, s0_std=0.05) if pair == "split"
         else _elu1(B=1, H=2, T=640, seed=5, s0_std=0.05))
    st = make_state(w.B, w.H, w.dk, w.dv, S=w.S0, xprev=w.xprev0)
    say(f"[znorm] {pair} pair, carried S0 and z0, in place")
    o, st2 = gpu_scan(w, S_in=st, S_out=st)
    o_ref, S_ref, z_ref, _ = oracle_scan(w)
    S, z, h = state_np(st2)
    eo, eS, ez = orc.relerr(o, o_ref), orc.relerr(S, S_ref), orc.relerr(z, z_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e} err(z)={ez:.3e}")
    assert eo <= TOL["bf16"] and eS <= TOL["bf16"] and ez <= TOL["bf16"]
    assert np.all(h == 1)


def test_znorm_scan_in_two_calls():
    """A scan cut at token 640 (the state, z included, handed from the first call to the
    second) matches the oracle over the whole sequence."""
    w = _identity(B=1, H=2, T=1000, seed=6)
    say("[znorm] two calls, cut at 640")
    o1, st = gpu_scan(w, t_slice=slice(0, 640))
    o2, st2 = gpu_scan(w, t_slice=slice(640, None), S_in=st)
    o_ref, S_ref, z_ref, _ = oracle_scan(w)
    o = np.concatenate([o1, o2], axis=2)
    S, z, _ = state_np(st2)
    eo, eS, ez = orc.relerr(o, o_ref), orc.relerr(S, S_ref), orc.relerr(z, z_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e} err(z)={ez:.3e}")
    assert eo <= TOL["bf16"] and eS <= TOL["bf16"] and ez <= TOL["bf16"]


@pytest.mark.parametrize("pair", ["split", "general"])
def test_znorm_segmented(pair):
    """One head of 8192 tokens: the library runs it as segments (virtual heads); the
    normaliser still chains over the real head's chunks."""
    w = _identity(B=1, H=1, T=8192, seed=7) if pair == "split" else _elu1(B=1, H=1, T=8192, seed=7)
    check_scan(w, label=f"znorm segmented {pair}")


def test_znorm_empty_scan_copies_state():
    import torch
    w = _identity(B=1, H=2, T=0, seed=8, s0_std=0.05)
    st_in = make_state(1, 2, 128, 128, S=w.S0, xprev=w.xprev0)
    st_out = F.State(1, 2, 128, 128)
    say("[znorm] T = 0")
    gpu_scan(w, S_in=st_in, S_out=st_out)
    torch.cuda.synchronize()
    S, z, _ = state_np(st_out)
    np.testing.assert_array_equal(S, w.S0.astype(np.float64))
    np.testing.assert_array_equal(z, w.xprev0.astype(np.float64))


@pytest.mark.parametrize("phi,pc,dtype,dk,dv", [
    ("elu1", False, "bf16", 128, 128),
    ("elu1", True, "f32", 64, 128),
    ("identity", False, "bf16", 128, 64),
    ("identity", True, "bf16", 64, 64),
])
def test_znorm_decode_sequence(phi, pc, dtype, dk, dv):
    """Several decode steps from a nonzero S0 and z0, in place after the first, against
    the oracle's step."""
    import torch
    B, H, steps = 3, 4, 6
    rng = np.random.default_rng(dk + dv + 7 * pc)
    S0 = (rng.standard_normal((B, H, dk, dv)) * 0.05).astype(np.float32)
    z0 = np.abs(rng.standard_normal((B, H, dk)) * 0.05).astype(np.float32)
    say(f"[znorm step] phi={phi} pc={pc} {dtype} dk={dk} dv={dv}")
    st_in = make_state(B, H, dk, dv, S=S0, xprev=z0)
    st = F.State(B, H, dk, dv)
    S_ref, z_ref, h_ref = S0.astype(np.float64), z0.astype(np.float64), None
    flags = F.ZNORM | (F.LAMBDA_PER_CHANNEL if pc else 0) | (F.PHI_ELU1 if phi == "elu1" else 0)
    bf = dtype == "bf16"

    def t(x, b):
        y = torch.from_numpy(np.ascontiguousarray(x))
        return (y.to(torch.bfloat16) if b else y).cuda()

    outs, refs = [], []
    for s in range(steps):
        q = rng.standard_normal((B, H, dk)).astype(np.float32)
        k = rng.standard_normal((B, H, dk)).astype(np.float32)
        if phi == "identity":
            q, k = np.abs(q), np.abs(k)
            q /= np.linalg.norm(q, axis=-1, keepdims=True)
            k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((B, H, dv)).astype(np.float32)
        if bf:
            q, k, v = wl.round_to_bf16(q), wl.round_to_bf16(k), wl.round_to_bf16(v)
        beta = rng.uniform(0.1, 1.0, size=(B, H)).astype(np.float32)
        lam = rng.uniform(0.8, 1.0, size=(B, H, dk) if pc else (B, H)).astype(np.float32)
        o, _ = F.step(t(q, bf), t(k, bf), t(v, bf), t(beta, False), t(lam, False),
                      rule=wl.RULE_ADDITIVE, flags=flags, eps=1e-6,
                      S_in=st_in if s == 0 else st, S_out=st)
        outs.append(o.cpu().numpy().astype(np.float64))
        o_ref, S_ref, z_ref, h_ref = orc.step(q, k, v, beta, lam, rule=wl.RULE_ADDITIVE,
                                              phi_kind=phi, eps=1e-6, per_channel=pc, S0=S_ref,
                                              xprev0=z_ref, has0=h_ref, znorm=True)
        refs.append(o_ref)
    torch.cuda.synchronize()
    S, z, h = state_np(st)
    eo, eS, ez = orc.relerr(np.stack(outs), np.stack(refs)), orc.relerr(S, S_ref), orc.relerr(z, z_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e} err(z)={ez:.3e}")
    assert eo <= TOL["f32"] and eS <= TOL["f32"] and ez <= TOL["f32"]
    assert np.all(h == 1)


def test_znorm_decode_with_qk_norm():
    """Decode with the normaliser and L2-normalised raw q, k (positive features)."""
    import torch
    B, H, d, steps = 2, 3, 128, 5
    rng = np.random.default_rng(77)
    st = F.State(B, H, d, d)
    S_ref = z_ref = h_ref = None
    outs, refs = [], []
    for s in range(steps):
        q, k = (np.abs(rng.standard_normal((B, H, d))).astype(np.float32) * 3 for _ in range(2))
        v = rng.standard_normal((B, H, d)).astype(np.float32)
        q, k, v = wl.round_to_bf16(q), wl.round_to_bf16(k), wl.round_to_bf16(v)
        lam = rng.uniform(0.8, 1.0, size=(B, H)).astype(np.float32)
        t = lambda x, b=True: (torch.from_numpy(x).to(torch.bfloat16) if b else torch.from_numpy(x)).cuda()
        o, _ = F.step(t(q), t(k), t(v), None, t(lam, False), rule=wl.RULE_ADDITIVE,
                      flags=F.ZNORM | F.QK_L2NORM, eps=1e-6, S_in=st if s else None, S_out=st)
        outs.append(o.cpu().numpy().astype(np.float64))
        o_ref, S_ref, z_ref, h_ref = orc.step(q, k, v, None, lam, rule=wl.RULE_ADDITIVE, eps=1e-6,
                                              S0=S_ref, xprev0=z_ref, has0=h_ref, qk_norm="l2",
                                              znorm=True)
        refs.append(o_ref)
    torch.cuda.synchronize()
    eo = orc.relerr(np.stack(outs), np.stack(refs))
    say(f"[znorm step qk-l2] err(o)={eo:.3e}")
    assert eo <= TOL["f32"]
