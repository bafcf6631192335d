"""The C-ABI library on the CPU: it loads, exports what include/fwmem.h declares, and
its host-side checks reject bad arguments before anything is launched (no GPU)."""
import ctypes
import os
import re

import pytest

from linear_attention_scan_amd import fwmem as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fwmem.h")


def _lib():
    if not os.path.exists(F.LIB_PATH):
        pytest.skip("libfwmem.so not built")
    return F.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fwmem_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(F.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_strerror():
    _lib()
    assert re.match(r"^\d+\.\d+\.\d+$", F.version())
    for code in (F.OK, F.EINVAL, F.EUNSUPPORTED, F.EALIGN, F.EOVERLAP, F.ELAUNCH, F.EWORKSPACE,
                 F.ESCRATCH, F.EWAIT):
        assert F.strerror(code) and F.strerror(code) != "unknown status"
    assert F.strerror(123) == "unknown status"


def test_state_and_workspace_sizes():
    _lib()
    B, H, dk, dv = 3, 5, 128, 64
    n = F.state_bytes(F.shape(B, H, 0, dk, dv, F.BF16))
    raw = 4 * (B * H * dk * dv + B * H * dk + B * H)
    assert n >= raw and n % 256 == 0 and n - raw < 256
    ws = F.workspace_bytes(F.shape(B, H, 130, dk, dv, F.BF16), F.mode())
    assert ws > 0 and ws % (B * H * 3) == 0          # 3 chunks of 64 for T = 130
    assert F.workspace_bytes(F.shape(B, H, 0, dk, dv, F.BF16), F.mode()) == 0
    ws32 = F.workspace_bytes(F.shape(B, H, 130, dk, dv, F.F32), F.mode())
    assert ws32 > ws                                  # fp32 operands take more room
    # the normaliser adds its chunk terms (132 + dk floats) and its value at each chunk entry
    wa = F.workspace_bytes(F.shape(B, H, 130, dk, dv, F.BF16), F.mode(rule=F.RULE_ADDITIVE))
    wz = F.workspace_bytes(F.shape(B, H, 130, dk, dv, F.BF16),
                           F.mode(rule=F.RULE_ADDITIVE, flags=F.ZNORM))
    al = lambda n: (n + 255) // 256 * 256
    assert wz == al(wa) + al(4 * B * H * 3 * (132 + dk)) + al(4 * B * H * 3 * dk)
    # the fused additive elu+1 kernel (bf16, scalar retention) keeps no records; segmented
    # (2 heads of T = 16384: 16 segments), it needs two virtual states and one float per segment
    assert F.workspace_bytes(F.shape(B, H, 130, dk, dv, F.BF16),
                             F.mode(rule=F.RULE_ADDITIVE, flags=F.PHI_ELU1)) == 0
    wseg = F.workspace_bytes(F.shape(1, 2, 16384, 128, 128, F.BF16),
                             F.mode(rule=F.RULE_ADDITIVE, flags=F.PHI_ELU1))
    VH = 2 * 16
    assert wseg == 2 * al(4 * (VH * 128 * 128 + VH * 128 + VH)) + al(4 * VH)


FAKE = 0x10000  # never dereferenced: every case below fails a host check first


def _scan(shp=None, md=None, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, lam=None, S_in=None, out=FAKE * 64,
          S_out=None, ws=FAKE * 128, ws_bytes=1 << 40):
    shp = shp or F.shape(1, 1, 8, 128, 128, F.BF16)
    md = md or F.mode()
    lib = _lib()
    return lib.fwmem_scan_fwd(ctypes.byref(shp), q, k, v, beta, lam, ctypes.byref(md), S_in, out,
                              S_out, ws, ws_bytes, None)


def _step(shp=None, md=None, q=FAKE, k=FAKE, v=FAKE, beta=FAKE, lam=None, S_in=None, out=FAKE * 64,
          S_out=FAKE * 1024):
    shp = shp or F.shape(1, 1, 1, 128, 128, F.BF16)
    md = md or F.mode()
    lib = _lib()
    return lib.fwmem_step(ctypes.byref(shp), q, k, v, beta, lam, ctypes.byref(md), S_in, out, S_out,
                          None)


@pytest.mark.parametrize("case,expect", [
    (dict(shp=F.shape(1, 1, 8, 96, 128, F.BF16)), F.EUNSUPPORTED),
    (dict(shp=F.shape(1, 1, 8, 128, 48, F.BF16)), F.EUNSUPPORTED),
    (dict(shp=F.shape(-1, 1, 8, 128, 128, F.BF16)), F.EINVAL),
    (dict(shp=F.shape(1, 1, -3, 128, 128, F.BF16)), F.EINVAL),
    (dict(shp=F.shape(1, 1, 8, 128, 128, 7)), F.EINVAL),
    (dict(md=F.mode(rule=5)), F.EINVAL),
    (dict(md=F.mode(flags=1 << 12)), F.EINVAL),
    (dict(md=F.mode(eps=-1.0)), F.EINVAL),
    (dict(md=F.mode(eps=float("nan"))), F.EINVAL),
    (dict(md=F.mode(chunk=48)), F.EUNSUPPORTED),
    (dict(q=None), F.EINVAL),
    (dict(out=None), F.EINVAL),
    (dict(beta=None), F.EINVAL),                      # delta rule needs beta
    (dict(beta=None, md=F.mode(rule=F.RULE_INNER)), F.EINVAL),  # so does the inner-product rule
    (dict(md=F.mode(rule=4)), F.EINVAL),
    # one step size per value channel takes a scalar ridge
    (dict(md=F.mode(rule=F.RULE_DELTA_PV, flags=F.LAMBDA_PER_CHANNEL)), F.EUNSUPPORTED),
    (dict(beta=None, md=F.mode(rule=F.RULE_DELTA_PV)), F.EINVAL),
    (dict(beta=FAKE + 4, md=F.mode(rule=F.RULE_DELTA_PV)), F.EALIGN),
    (dict(md=F.mode(flags=F.QK_L2NORM | F.QK_RMSNORM)), F.EINVAL),
    (dict(md=F.mode(flags=F.QK_RMSNORM | F.PHI_ELU1)), F.EUNSUPPORTED),
    (dict(md=F.mode(flags=F.BETA_SIGMOID | F.BETA_SIGMOID2)), F.EINVAL),
    # the normaliser takes the additive rule, and scans a scalar decay and float32 outputs
    (dict(md=F.mode(flags=F.ZNORM)), F.EUNSUPPORTED),
    (dict(md=F.mode(rule=F.RULE_INNER, flags=F.ZNORM)), F.EUNSUPPORTED),
    (dict(md=F.mode(rule=F.RULE_ADDITIVE, flags=F.ZNORM | F.LAMBDA_PER_CHANNEL)), F.EUNSUPPORTED),
    (dict(md=F.mode(rule=F.RULE_ADDITIVE, flags=F.ZNORM | F.OUT_BF16)), F.EUNSUPPORTED),
    # the scale-coupled ridge: a ridge (delta, inner), and in scans a scalar one
    (dict(md=F.mode(rule=F.RULE_ADDITIVE, flags=F.LAMBDA_SCALED)), F.EUNSUPPORTED),
    (dict(md=F.mode(flags=F.LAMBDA_SCALED | F.LAMBDA_PER_CHANNEL)), F.EUNSUPPORTED),
    (dict(q=FAKE + 2), F.EALIGN),
    (dict(out=FAKE * 64 + 8), F.EALIGN),
    (dict(beta=FAKE + 2), F.EALIGN),
    (dict(md=F.mode(flags=F.LAMBDA_PER_CHANNEL), lam=FAKE + 4), F.EALIGN),
    (dict(S_in=FAKE * 4096, S_out=FAKE * 4096 + 256), F.EOVERLAP),
    (dict(out=FAKE, q=FAKE), F.EOVERLAP),             # out on top of q
    (dict(ws=FAKE * 64), F.EOVERLAP),                 # workspace on top of out
    (dict(ws=None), F.EWORKSPACE),
    (dict(ws_bytes=16), F.EWORKSPACE),
])
def test_scan_rejects(case, expect):
    assert _scan(**case) == expect


def test_scan_null_shape_and_mode():
    lib = _lib()
    md = F.mode()
    shp = F.shape(1, 1, 8, 128, 128, F.BF16)
    assert lib.fwmem_scan_fwd(None, FAKE, FAKE, FAKE, FAKE, None, ctypes.byref(md), None, FAKE * 64,
                              None, FAKE * 128, 1 << 40, None) == F.EINVAL
    assert lib.fwmem_scan_fwd(ctypes.byref(shp), FAKE, FAKE, FAKE, FAKE, None, None, None,
                              FAKE * 64, None, FAKE * 128, 1 << 40, None) == F.EINVAL


def test_empty_batch_is_a_no_op():
    # B*H == 0: nothing to do, no pointer is needed
    assert _scan(shp=F.shape(0, 4, 8, 128, 128, F.BF16), q=None, k=None, v=None, out=None,
                 ws=None) == F.OK
    assert _step(shp=F.shape(3, 0, 1, 64, 64, F.F32), q=None, out=None, S_out=None) == F.OK


@pytest.mark.parametrize("case,expect", [
    (dict(shp=F.shape(1, 1, 1, 128, 32, F.BF16)), F.EUNSUPPORTED),
    (dict(S_out=None), F.EINVAL),
    (dict(beta=None), F.EINVAL),
    (dict(beta=None, md=F.mode(rule=F.RULE_INNER)), F.EINVAL),
    (dict(md=F.mode(rule=-1)), F.EINVAL),
    (dict(md=F.mode(rule=F.RULE_ADDITIVE, flags=1 << 12)), F.EINVAL),
    (dict(md=F.mode(rule=F.RULE_DELTA, flags=F.ZNORM)), F.EUNSUPPORTED),
    (dict(md=F.mode(rule=F.RULE_DELTA_PV, flags=F.LAMBDA_PER_CHANNEL)), F.EUNSUPPORTED),
    (dict(beta=None, md=F.mode(rule=F.RULE_DELTA_PV)), F.EINVAL),
    (dict(md=F.mode(rule=F.RULE_ADDITIVE, flags=F.LAMBDA_SCALED)), F.EUNSUPPORTED),
    (dict(q=FAKE + 1), F.EALIGN),
    (dict(out=FAKE * 64 + 4), F.EALIGN),
    (dict(S_in=FAKE * 1024 + 64), F.EOVERLAP),
    (dict(out=FAKE * 1024), F.EOVERLAP),
])
def test_step_rejects(case, expect):
    assert _step(**case) == expect


M = 1 << 24  # backward cases: every buffer 16 MiB from the next, none dereferenced


def _bwd(shp=None, md=None, q=M, k=2 * M, v=3 * M, beta=4 * M, lam=None, S_in=None, gout=5 * M,
         gSout=None, gq=6 * M, gk=7 * M, gv=8 * M, gbeta=9 * M, glam=None, gSin=10 * M, ws=11 * M,
         ws_bytes=1 << 40):
    shp = shp or F.shape(1, 1, 8, 128, 128, F.BF16)
    md = md or F.mode()
    lib = _lib()
    return lib.fwmem_scan_bwd(ctypes.byref(shp), q, k, v, beta, lam, ctypes.byref(md), S_in, gout,
                              gSout, gq, gk, gv, gbeta, glam, gSin, ws, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    (dict(shp=F.shape(1, 1, 8, 96, 128, F.BF16)), F.EUNSUPPORTED),
    (dict(md=F.mode(rule=F.RULE_DELTA_PV, flags=F.LAMBDA_PER_CHANNEL)), F.EUNSUPPORTED),
    (dict(md=F.mode(rule=F.RULE_DELTA_PV, flags=F.ZNORM)), F.EUNSUPPORTED),
    (dict(md=F.mode(rule=F.RULE_DELTA_PV), gbeta=9 * M + 4), F.EALIGN),   # per-column beta: float4
    (dict(md=F.mode(rule=F.RULE_DELTA_PV), gbeta=4 * M + 64), F.EOVERLAP),  # onto beta [.., dv]
    (dict(md=F.mode(flags=F.OUT_BF16)), F.EUNSUPPORTED),
    (dict(md=F.mode(flags=F.LAMBDA_SCALED | F.LAMBDA_PER_CHANNEL)), F.EUNSUPPORTED),
    (dict(md=F.mode(rule=F.RULE_ADDITIVE, flags=F.LAMBDA_SCALED)), F.EUNSUPPORTED),
    (dict(md=F.mode(flags=F.QK_L2NORM | F.PHI_ELU1)), F.EUNSUPPORTED),
    (dict(md=F.mode(rule=F.RULE_ADDITIVE, flags=F.ZNORM | F.LAMBDA_PER_CHANNEL)), F.EUNSUPPORTED),
    (dict(md=F.mode(rule=F.RULE_ADDITIVE, flags=F.ZNORM | F.OUT_BF16)), F.EUNSUPPORTED),
    (dict(md=F.mode(flags=1 << 12)), F.EINVAL),
    (dict(md=F.mode(rule=7)), F.EINVAL),
    (dict(beta=None), F.EINVAL),
    (dict(gout=None), F.EINVAL),
    (dict(gq=None), F.EINVAL),
    (dict(gv=None), F.EINVAL),
    (dict(ws=None), F.EWORKSPACE),
    (dict(ws_bytes=4096), F.EWORKSPACE),
    (dict(gv=8 * M + 4), F.EALIGN),
    (dict(ws=11 * M + 8), F.EALIGN),
    (dict(gSin=10 * M + 4), F.EALIGN),
    (dict(gq=1 * M), F.EOVERLAP),         # onto q
    (dict(gk=6 * M + 64), F.EOVERLAP),    # onto grad_q
    (dict(ws=8 * M), F.EOVERLAP),         # onto grad_v
    (dict(gbeta=4 * M), F.EOVERLAP),      # onto beta
])
def test_bwd_rejects(case, expect):
    assert _bwd(**case) == expect


def test_bwd_workspace_size_and_empty_batch():
    lib = _lib()
    n = ctypes.c_size_t(0)
    shp, md = F.shape(2, 3, 100, 128, 64, F.F32), F.mode(rule=F.RULE_INNER)
    assert lib.fwmem_scan_bwd_workspace_bytes(ctypes.byref(shp), ctypes.byref(md), ctypes.byref(n)) == F.OK
    # the chunk-parallel backward (scalar decay, no normaliser): per 64-token chunk one
    # record of 13,184 floats (three 64x64 matrices, 13 rows of per-token scalars and one
    # row of chunk values, padded to a multiple of 64), two d_k x d_v states and two
    # 64 x d_v blocks
    want = 4 * 6 * 2 * (13184 + 2 * 128 * 64 + 2 * 64 * 64)
    assert n.value == (want + 255) // 256 * 256
    # the per-value-channel rule: 32-token chunks as well
    mdv = F.mode(rule=F.RULE_DELTA_PV)
    assert lib.fwmem_scan_bwd_workspace_bytes(ctypes.byref(shp), ctypes.byref(mdv), ctypes.byref(n)) == F.OK
    want = 4 * 6 * ((4 + 32) * 128 * 64 + 32 * 64)
    assert n.value == (want + 255) // 256 * 256
    # the normaliser: 32-token chunks and its value at each chunk start
    mdz = F.mode(rule=F.RULE_ADDITIVE, flags=F.ZNORM)
    assert lib.fwmem_scan_bwd_workspace_bytes(ctypes.byref(shp), ctypes.byref(mdz), ctypes.byref(n)) == F.OK
    want = 4 * 6 * ((4 + 32) * 128 * 64 + 32 * 64 + 4 * 128)
    assert n.value == (want + 255) // 256 * 256
    shp0 = F.shape(2, 3, 0, 128, 64, F.F32)
    assert lib.fwmem_scan_bwd_workspace_bytes(ctypes.byref(shp0), ctypes.byref(md), ctypes.byref(n)) == F.OK
    assert n.value == 0
    assert lib.fwmem_scan_bwd_workspace_bytes(ctypes.byref(shp), ctypes.byref(md), None) == F.EINVAL
    # per-channel lambda: 32-token chunks
    mdp = F.mode(rule=F.RULE_INNER, flags=F.LAMBDA_PER_CHANNEL)
    assert lib.fwmem_scan_bwd_workspace_bytes(ctypes.byref(shp), ctypes.byref(mdp), ctypes.byref(n)) == F.OK
    want = 4 * 6 * ((4 + 32) * 128 * 64 + 32 * 64)
    assert n.value == (want + 255) // 256 * 256
    # B*H == 0: nothing to do, no pointer is needed
    assert _bwd(shp=F.shape(0, 2, 8, 64, 64, F.F32), q=None, k=None, v=None, gout=None, gq=None,
                gk=None, gv=None, ws=None) == F.OK


def test_noalloc_rejects_a_workspace_beyond_its_scratch():
    # host-side check, before any device call: 64 bf16 heads of T = 4096 at d = 128 need
    # about 107 MB of workspace, beyond the 64 MiB scratch
    _lib()
    shp = F.shape(4, 16, 4096, 128, 128, F.BF16)
    md = F.mode(F.RULE_DELTA, 0, 1e-6, 0)
    assert F.workspace_bytes(shp, md) > F.NOALLOC_SCRATCH_BYTES
    st = F.scan_fwd_noalloc_raw(shp, 16, 16, 16, 16, 16, md, None, 16, None, stream=0)
    assert st == F.ESCRATCH
    # argument errors come first, as for fwmem_scan_fwd
    bad = F.mode(7, 0, 1e-6, 0)
    assert F.scan_fwd_noalloc_raw(shp, 16, 16, 16, 16, 16, bad, None, 16, None, stream=0) == F.EINVAL
