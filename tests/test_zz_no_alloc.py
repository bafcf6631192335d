"""fwmem_scan_fwd_noalloc (the scan on the library's fixed device scratch) against
fwmem_scan_fwd (the scan on a caller workspace), through the C ABI: two calls in a row,
the second on a smaller input, each equal to the workspace entry point's result and
within the oracle's tolerance."""
import numpy as np
import pytest
import torch

from linear_attention_scan_amd import fwmem as F
from linear_attention_scan_amd import workloads as wl
from oracle import fwmem_oracle as orc
from tests.gpu_helpers import TOL, dev_tensor, f32_tensor, say

pytestmark = pytest.mark.gpu


def _flags(w):
    return (F.PHI_ELU1 if w.phi == wl.PHI_ELU1 else 0) | (F.LAMBDA_PER_CHANNEL if w.per_channel else 0)


def _both(w):
    """Run w through both entry points on the same device inputs; returns the two
    (out, S_out) pairs as host arrays."""
    q, k, v = (dev_tensor(x, w.dtype) for x in (w.q, w.k, w.v))
    beta, lam = f32_tensor(w.beta), f32_tensor(w.lam)
    shp = F.shape(w.B, w.H, w.T, w.dk, w.dv, F.BF16 if w.dtype == "bf16" else F.F32)
    md = F.mode(w.rule, _flags(w), w.eps, 0)
    need = F.workspace_bytes(shp, md)
    assert 0 < need <= F.NOALLOC_SCRATCH_BYTES
    res = []
    for noalloc in (False, True):
        out = torch.full((w.B, w.H, w.T, w.dv), float("nan"), dtype=torch.float32, device="cuda")
        S_out = F.State(w.B, w.H, w.dk, w.dv)
        S_out.buf.fill_(float("nan"))
        if noalloc:
            st = F.scan_fwd_noalloc_raw(shp, q, k, v, beta, lam, md, None, out, S_out.buf)
        else:
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            st = F.scan_fwd_raw(shp, q, k, v, beta, lam, md, None, out, S_out.buf, ws, need)
        assert st == F.OK, F.strerror(st)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), S_out.S.cpu().numpy(), S_out.x_prev.cpu().numpy(),
                    S_out.has_prev.cpu().numpy()))
    return res


def test_noalloc_matches_the_workspace_entry_point_twice():
    # the first call fills more of the scratch than the second: a delta-rule scan on the
    # split pair, then a smaller delta-rule elu+1 scan (general pair, other head sizes)
    cases = [wl.delta_bf16(seed=0, B=2, H=4, T=1000),
             wl.make_scan(B=1, H=2, T=130, dk=64, dv=128, dtype="bf16", phi=wl.PHI_ELU1,
                          beta_kind="sigmoid", lam_kind="softplus", normalise_qk=False, seed=3)]
    sizes = []
    for w in cases:
        say(f"noalloc: rule {w.rule} B{w.B} H{w.H} T{w.T} dk{w.dk} dv{w.dv}")
        (o_ws, S_ws, x_ws, h_ws), (o_na, S_na, x_na, h_na) = _both(w)
        # the same kernels on the same inputs: bit-identical results
        assert np.array_equal(o_ws, o_na) and np.array_equal(S_ws, S_na)
        assert np.array_equal(x_ws, x_na) and np.array_equal(h_ws, h_na)
        o_ref, S_ref, _, _ = orc.scan(w.q, w.k, w.v, w.beta, w.lam, rule=w.rule, phi_kind=w.phi,
                                      eps=w.eps, per_channel=w.per_channel)
        tol = TOL[w.dtype]
        assert orc.relerr(o_na, o_ref) <= tol and orc.relerr(S_na, S_ref) <= tol
        shp = F.shape(w.B, w.H, w.T, w.dk, w.dv, F.BF16)
        sizes.append(F.workspace_bytes(shp, F.mode(w.rule, _flags(w), w.eps, 0)))
    assert sizes[1] < sizes[0]


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    # B*H = 64 heads of T = 4096 (bf16 delta rule, d = 128) need about 107 MB
    shp = F.shape(4, 16, 4096, 128, 128, F.BF16)
    md = F.mode(F.RULE_DELTA, 0, 1e-6, 0)
    assert F.workspace_bytes(shp, md) > F.NOALLOC_SCRATCH_BYTES
    st = F.scan_fwd_noalloc_raw(shp, 16, 16, 16, 16, 16, md, None, 16, None, stream=0)
    assert st == F.ESCRATCH
