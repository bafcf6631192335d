"""Helpers for the GPU parity tests: run a workload through libfwmem (via the C ABI)
and through the fp64 oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np

from linear_attention_scan_amd import fwmem as F
from linear_attention_scan_amd import workloads as wl
from oracle import fwmem_oracle as orc

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_tensor(x, dtype_name):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype_name == "bf16":
        t = t.to(torch.bfloat16)
    return t.to("cuda")


def f32_tensor(x):
    import torch
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def flags_of(w: wl.ScanInputs, extra=0):
    f = extra
    if w.phi == wl.PHI_ELU1:
        f |= F.PHI_ELU1
    if w.per_channel:
        f |= F.LAMBDA_PER_CHANNEL
    if w.qk_norm is not None:
        f |= {"l2": F.QK_L2NORM, "rms": F.QK_RMSNORM}[w.qk_norm]
    if w.gates_pre:
        if w.beta_act is not None:
            f |= {"sigmoid": F.BETA_SIGMOID, "sigmoid2": F.BETA_SIGMOID2}[w.beta_act]
        if w.lam_act:
            f |= F.LAMBDA_PREACT
    if w.znorm:
        f |= F.ZNORM
    if w.lam_scaled:
        f |= F.LAMBDA_SCALED
    return f


def gates_of(w: wl.ScanInputs):
    """The gate arrays the library receives: the activated gates, or with gates_pre the
    pre-activations they were drawn from (those that have one)."""
    beta = w.beta_pre if (w.gates_pre and w.beta_act is not None) else w.beta
    lam = w.lam_pre if (w.gates_pre and w.lam_act) else w.lam
    return beta, lam


def make_state(B, H, dk, dv, S=None, xprev=None, has=None):
    import torch
    st = F.State(B, H, dk, dv)
    if S is not None:
        st.S.copy_(torch.from_numpy(np.ascontiguousarray(S, dtype=np.float32)))
    if xprev is not None:
        st.x_prev.copy_(torch.from_numpy(np.ascontiguousarray(xprev, dtype=np.float32)))
    if has is not None:
        st.has_prev.copy_(torch.from_numpy(np.ascontiguousarray(has, dtype=np.int32)))
    return st


def gpu_scan(w: wl.ScanInputs, *, t_slice=None, S_in=None, S_out=None, extra_flags=0):
    """Run fwmem_scan_fwd on w (optionally on tokens t_slice only). Returns
    (out [B,H,T,dv] float64, State)."""
    import torch
    sl = slice(None) if t_slice is None else t_slice
    q = dev_tensor(w.q[:, :, sl], w.dtype)
    k = dev_tensor(w.k[:, :, sl], w.dtype)
    v = dev_tensor(w.v[:, :, sl], w.dtype)
    gb, gl = gates_of(w)
    beta = f32_tensor(None if gb is None else gb[:, :, sl])
    lam = f32_tensor(None if gl is None else gl[:, :, sl])
    if S_in is None and w.S0 is not None:
        S_in = make_state(w.B, w.H, w.dk, w.dv, S=w.S0, xprev=w.xprev0, has=w.has0)
    out, st = F.scan_fwd(q, k, v, beta, lam, rule=w.rule, flags=flags_of(w, extra_flags),
                         eps=w.eps, S_in=S_in, S_out=S_out)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), st


def oracle_scan(w: wl.ScanInputs, t_slice=None, S0=None, xprev0=None, has0=None):
    sl = slice(None) if t_slice is None else t_slice
    S0 = w.S0 if S0 is None else S0
    xprev0 = w.xprev0 if xprev0 is None else xprev0
    has0 = w.has0 if has0 is None else has0
    gb, gl = gates_of(w)
    return orc.scan(w.q[:, :, sl], w.k[:, :, sl], w.v[:, :, sl],
                    None if gb is None else gb[:, :, sl],
                    None if gl is None else gl[:, :, sl],
                    rule=w.rule, phi_kind=w.phi, eps=w.eps, per_channel=w.per_channel,
                    S0=S0, xprev0=xprev0, has0=has0, qk_norm=w.qk_norm,
                    beta_act=w.beta_act if (w.gates_pre and gb is w.beta_pre) else None,
                    lam_act=bool(w.gates_pre and w.lam_act), znorm=w.znorm,
                    lam_scaled=w.lam_scaled)


def state_np(st):
    return (st.S.cpu().numpy().astype(np.float64), st.x_prev.cpu().numpy().astype(np.float64),
            st.has_prev.cpu().numpy())


def check_scan(w: wl.ScanInputs, tol=None, label=""):
    """Full parity of one workload: o and final S within tol; x_prev and has_prev exact."""
    tol = TOL[w.dtype] if tol is None else tol
    say(f"[scan] {label or w.name} B={w.B} H={w.H} T={w.T} dk={w.dk} dv={w.dv} {w.dtype} "
        f"rule={w.rule} phi={w.phi} pc={w.per_channel}")
    o, st = gpu_scan(w)
    o_ref, S_ref, x_ref, h_ref = oracle_scan(w)
    S, x, h = state_np(st)
    eo, eS = orc.relerr(o, o_ref), orc.relerr(S, S_ref)
    say(f"    err(o)={eo:.3e} err(S)={eS:.3e} tol={tol:g}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    assert eo <= tol, f"err(o)={eo}"
    assert eS <= tol, f"err(S)={eS}"
    if w.znorm:  # the slot holds the normaliser z
        ex = orc.relerr(x, x_ref)
        say(f"    err(z)={ex:.3e}")
        assert ex <= tol, f"err(z)={ex}"
        assert w.T == 0 or np.all(h == 1)
    elif w.T > 0:
        if w.phi == wl.PHI_IDENTITY:
            np.testing.assert_array_equal(x, x_ref.astype(np.float32).astype(np.float64))
        else:  # elu+1 is evaluated in fp32 on the GPU
            np.testing.assert_allclose(x, x_ref, rtol=4e-6, atol=1e-30)
        assert np.all(h == 1)
    return eo, eS
