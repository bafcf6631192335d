"""The device status word of the split propagate kernel's bounded waits: a scan whose
waits are forced (from the host, by the test hook FWMEM_TEST_WAIT_TIMEOUT) to give up
after a few polls still finishes, and fwmem_check_device reports FWMEM_EWAIT once, then
FWMEM_OK; an ordinary scan afterwards is correct and reports nothing."""
import pytest
import torch

from linear_attention_scan_amd import fwmem as F
from linear_attention_scan_amd import workloads as wl
from oracle import fwmem_oracle as orc
from tests.gpu_helpers import TOL, dev_tensor, f32_tensor, say

pytestmark = pytest.mark.gpu


def _scan(w):
    out, st = F.scan_fwd(dev_tensor(w.q, w.dtype), dev_tensor(w.k, w.dtype),
                         dev_tensor(w.v, w.dtype), f32_tensor(w.beta), f32_tensor(w.lam),
                         rule=w.rule, eps=w.eps)
    return out, st


def test_a_wait_that_gives_up_is_reported(monkeypatch):
    w = wl.delta_bf16(seed=0, B=1, H=2, T=300)
    say("status: clean start")
    assert F.check_device() == F.OK
    monkeypatch.setenv("FWMEM_TEST_WAIT_TIMEOUT", "4")
    say("status: scan with every wait forced to give up after 4 polls")
    _scan(w)
    assert F.check_device() == F.EWAIT
    assert F.check_device() == F.OK  # read once, then cleared
    monkeypatch.delenv("FWMEM_TEST_WAIT_TIMEOUT")
    say("status: ordinary scan")
    out, st = _scan(w)
    assert F.check_device() == F.OK
    o_ref, S_ref, _, _ = orc.scan(w.q, w.k, w.v, w.beta, w.lam, rule=w.rule, eps=w.eps)
    assert orc.relerr(out.cpu().numpy(), o_ref) <= TOL["bf16"]
    assert orc.relerr(st.S.cpu().numpy(), S_ref) <= TOL["bf16"]
    torch.cuda.synchronize()
