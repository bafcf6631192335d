#!/usr/bin/env python3
"""Throughput of libfwmem on one MI355X.

A step is one pass of the whole scan (the chunk-prep kernel, then the propagate
kernel: exactly fwmem_scan_fwd) over one batch of synthetic input already resident
in HBM. The default workload is the delta rule at B=4, H=16, T=4096, d_k=d_v=128
with bf16 q/k/v (beta = 2 sigmoid(N(0,1)), lambda = softplus(N(-4,1)), seed 0).

Prints ONE JSON line. `value` comes from K steps timed back to back; `roofline` is for
the longer of the two kernels, from HIP events recorded around every launch of a second
run of K steps, on the stream the kernels run on. The decode kernel (fwmem_step at
B=256, H=32, d=128) is measured in the same run and reported under `decode`, and the
backward pass (fwmem_scan_bwd) on the same workload, where it supports the workload's
mode, under `backward`.
`cpu_baseline` is the fp64 oracle timed on the host (a bounded sample of the same
workload: whole batch elements, about 10 s).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fast-weight scan tokens/s per GPU (H=16,d=128,T=4096) + % MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "linear_attention_scan_amd", "csrc")

# HBM traffic per launch of the scan kernels and the chunk-parallel backward's kernels on the
# default workload (B=4 H=16 T=4096 d=128, bf16, delta rule) and of the decode kernel
# (B=256 H=32 d=128, state in place),
# from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE in runs of their own, each scaled by
# what the same counter reads for a plain 1 GiB device copy in the same run
# (FETCH_SIZE x2.0, WRITE_SIZE x1.0). A record is reported only while the
# kernel's sources still hash to the recorded digest; after any change it is null until
# the counters are taken again.
MEASURED_TRAFFIC = {
    ("delta_bf16_h16", "prop_split_kernel"): {
        "sources": ('fwmem_scan_split.hip', 'fwmem_split.h', 'fwmem_device.h', 'fwmem_internal.h'),
        "sha256": {
            "fwmem_scan_split.hip": "8dad3d6f246efa0358bc68fa1ca0969768f0cbb50970ea006490d38df3a1dcf9",
            "fwmem_split.h": "4591e7fd7055f318ad39f2d4e4db57e3d0fc5b48fefc454192d92052048145be",
            "fwmem_device.h": "90ffc6ed9c432872bfbb7f5721e8afbed17fcc7efdc6a739875472e513370cd9",
            "fwmem_internal.h": "033dab365d38d3acdac54d3b0c36484685eff444330d782d2e2eff68dba2abf0",
        },
        "fetch_kib": 150222.5, "write_kib": 135202.0, "read_factor": 2.0, "write_factor": 1.0,
    },
    ("delta_bf16_h16", "prep_split_kernel"): {
        "sources": ('fwmem_prep_split.hip', 'fwmem_split.h', 'fwmem_device.h', 'fwmem_internal.h'),
        "sha256": {
            "fwmem_prep_split.hip": "3101a25cff5f80c14678715ef955e7813e5203414cf5f028e6a8e885c74a10f8",
            "fwmem_split.h": "4591e7fd7055f318ad39f2d4e4db57e3d0fc5b48fefc454192d92052048145be",
            "fwmem_device.h": "90ffc6ed9c432872bfbb7f5721e8afbed17fcc7efdc6a739875472e513370cd9",
            "fwmem_internal.h": "033dab365d38d3acdac54d3b0c36484685eff444330d782d2e2eff68dba2abf0",
        },
        "fetch_kib": 66681.6, "write_kib": 103566.0, "read_factor": 2.0, "write_factor": 1.0,
    },
    ("decode", "step_kernel"): {
        "sources": ('fwmem_step.hip', 'fwmem_device.h', 'fwmem_internal.h'),
        "sha256": {
            "fwmem_step.hip": "abf27317cda12cc5a31bfd56f61be55aedc5758d577a0abf5f1d25a096ca1990",
            "fwmem_device.h": "90ffc6ed9c432872bfbb7f5721e8afbed17fcc7efdc6a739875472e513370cd9",
            "fwmem_internal.h": "033dab365d38d3acdac54d3b0c36484685eff444330d782d2e2eff68dba2abf0",
        },
        "fetch_kib": 267738.2, "write_kib": 532870.6, "read_factor": 2.0, "write_factor": 1.0,
    },
    ("delta_bf16_h16", "bwd_prep_kernel"): {
        "sources": ('fwmem_backward_chunk.hip', 'fwmem_backward.h', 'fwmem_split.h', 'fwmem_device.h', 'fwmem_internal.h'),
        "sha256": {
            "fwmem_backward_chunk.hip": "43a1c156089b10bfe6ac36cfe3d57721a366030ccd20b0939aaf8266446dc921",
            "fwmem_backward.h": "a5fd0f8c1f47a680f2609b5378a6eaef440ead7d30c31d73b985adaf1ed93a10",
            "fwmem_split.h": "4591e7fd7055f318ad39f2d4e4db57e3d0fc5b48fefc454192d92052048145be",
            "fwmem_device.h": "90ffc6ed9c432872bfbb7f5721e8afbed17fcc7efdc6a739875472e513370cd9",
            "fwmem_internal.h": "033dab365d38d3acdac54d3b0c36484685eff444330d782d2e2eff68dba2abf0",
        },
        "fetch_kib": 66695.4, "write_kib": 210048.0, "read_factor": 2.0, "write_factor": 1.0,
    },
    ("delta_bf16_h16", "bwd_state_bf_kernel"): {
        "sources": ('fwmem_backward_chunk.hip', 'fwmem_backward.h', 'fwmem_split.h', 'fwmem_device.h', 'fwmem_internal.h'),
        "sha256": {
            "fwmem_backward_chunk.hip": "43a1c156089b10bfe6ac36cfe3d57721a366030ccd20b0939aaf8266446dc921",
            "fwmem_backward.h": "a5fd0f8c1f47a680f2609b5378a6eaef440ead7d30c31d73b985adaf1ed93a10",
            "fwmem_split.h": "4591e7fd7055f318ad39f2d4e4db57e3d0fc5b48fefc454192d92052048145be",
            "fwmem_device.h": "90ffc6ed9c432872bfbb7f5721e8afbed17fcc7efdc6a739875472e513370cd9",
            "fwmem_internal.h": "033dab365d38d3acdac54d3b0c36484685eff444330d782d2e2eff68dba2abf0",
        },
        "fetch_kib": 100195.2, "write_kib": 393216.0, "read_factor": 2.0, "write_factor": 1.0,
    },
    ("delta_bf16_h16", "bwd_dstate_bf_kernel"): {
        "sources": ('fwmem_backward_chunk.hip', 'fwmem_backward.h', 'fwmem_split.h', 'fwmem_device.h', 'fwmem_internal.h'),
        "sha256": {
            "fwmem_backward_chunk.hip": "43a1c156089b10bfe6ac36cfe3d57721a366030ccd20b0939aaf8266446dc921",
            "fwmem_backward.h": "a5fd0f8c1f47a680f2609b5378a6eaef440ead7d30c31d73b985adaf1ed93a10",
            "fwmem_split.h": "4591e7fd7055f318ad39f2d4e4db57e3d0fc5b48fefc454192d92052048145be",
            "fwmem_device.h": "90ffc6ed9c432872bfbb7f5721e8afbed17fcc7efdc6a739875472e513370cd9",
            "fwmem_internal.h": "033dab365d38d3acdac54d3b0c36484685eff444330d782d2e2eff68dba2abf0",
        },
        "fetch_kib": 199003.4, "write_kib": 397314.0, "read_factor": 2.0, "write_factor": 1.0,
    },
    ("delta_bf16_h16", "bwd_grad_kernel"): {
        "sources": ('fwmem_backward_chunk.hip', 'fwmem_backward.h', 'fwmem_split.h', 'fwmem_device.h', 'fwmem_internal.h'),
        "sha256": {
            "fwmem_backward_chunk.hip": "43a1c156089b10bfe6ac36cfe3d57721a366030ccd20b0939aaf8266446dc921",
            "fwmem_backward.h": "a5fd0f8c1f47a680f2609b5378a6eaef440ead7d30c31d73b985adaf1ed93a10",
            "fwmem_split.h": "4591e7fd7055f318ad39f2d4e4db57e3d0fc5b48fefc454192d92052048145be",
            "fwmem_device.h": "90ffc6ed9c432872bfbb7f5721e8afbed17fcc7efdc6a739875472e513370cd9",
            "fwmem_internal.h": "033dab365d38d3acdac54d3b0c36484685eff444330d782d2e2eff68dba2abf0",
        },
        "fetch_kib": 629742.6, "write_kib": 395396.3, "read_factor": 2.0, "write_factor": 1.0,
    },
}


def measured_traffic(workload, kernel):
    """Calibrated HBM bytes per launch from the counter record, or None when there is no
    record or the kernel's sources have changed since it was taken."""
    import hashlib
    rec = MEASURED_TRAFFIC.get((workload, kernel))
    if rec is None:
        return None
    for name in rec["sources"]:
        try:
            with open(os.path.join(CSRC, name), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != rec["sha256"][name]:
                    return None
        except OSError:
            return None
    return int(round(rec["fetch_kib"] * 1024 * rec["read_factor"]
                     + rec["write_kib"] * 1024 * rec["write_factor"]))


def kernel_names(w):
    """Names of the prep and propagate kernels that the library launches for w: bf16
    inputs with the identity feature map and a scalar decay take the split-operand
    kernels; the additive rule with elu+1 on bf16 (scalar retention) one fused kernel in
    the propagate phase (its prep phase only sets up segments); everything else the
    general ones; the per-value-channel rule its own (state and solver waves for bf16 with
    the identity map)."""
    if w.rule == 3:
        pv2 = w.dtype == "bf16" and w.phi != "elu1"
        return {"prep": "prep_pv_kernel", "propagate": "prop_pv2_kernel" if pv2 else "prop_pv_kernel"}
    if w.rule == 1 and w.dtype == "bf16" and w.phi == "elu1" and not w.per_channel:
        return {"prep": "seg_init_kernel", "propagate": "add_kernel"}
    split = w.dtype == "bf16" and not w.per_channel and w.phi != "elu1"
    return ({"prep": "prep_split_kernel", "propagate": "prop_split_kernel"} if split
            else {"prep": "prep_kernel", "propagate": "prop_kernel"})


def compute_dtype(w):
    """Arithmetic type of the scan: the split kernels, the fused additive kernel and the
    per-value-channel state and solver waves multiply bf16 operands (hi/lo pairs for
    computed matrices), the general kernels fp16 operands for bf16 inputs, fp32 inputs
    (and the per-value-channel rule on them) fp32 operands; all accumulate in fp32."""
    if w.dtype != "bf16":
        return "f32"
    prop = kernel_names(w)["propagate"]
    if w.rule == 3:
        return "bf16" if prop == "prop_pv2_kernel" else "f32"
    return "bf16" if prop in ("prop_split_kernel", "add_kernel") else "f16"


def scan_bytes_per_token_head(w, out_bytes=4):
    """HBM bytes of the scan per (token, head) with o written as float32 (the library's
    default output): q, k, v read once, beta and lambda read once, out written once (the
    state adds d_k*d_v*8 per head per call)."""
    es = 2 if w.dtype == "bf16" else 4
    lam = 0 if w.lam is None else 4 * (w.dk if w.per_channel else 1)
    beta = 0 if w.beta is None else 4 * (w.dv if w.rule == 3 else 1)
    return (2 * w.dk + w.dv) * es + beta + lam + w.dv * out_bytes


def algorithmic_bytes_per_token_head(w):
    """Algorithmic HBM bytes per (token, head) as the hot-path scope table counts them:
    q, k, v read once and o written once, all in the input type (3d*s + d*s), plus the
    float32 gates (4 for a scalar gate, 4*d_k for a per-channel lambda, 4*d_v for a
    per-value-channel beta). At d = 128 with bf16 inputs and both gates: 1032 B."""
    es = 2 if w.dtype == "bf16" else 4
    return scan_bytes_per_token_head(w, out_bytes=es)


def algorithmic_flops_per_token_head(w, C=64):
    """Flops per (token, head) of the chunked form, counting only the triangular halves of
    the in-chunk products: 3 C d_k + 2 C d_v + 6 d_k d_v with the delta rule's solve, and
    C (d_k + d_v) + 4 d_k d_v without one (additive and inner-product rules)."""
    if w.rule in (0, 3):
        return 3 * C * w.dk + 2 * C * w.dv + 6 * w.dk * w.dv
    return C * (w.dk + w.dv) + 4 * w.dk * w.dv


def executed_flops_per_token_head(w, C=64):
    """MFMA flops per (token, head) that the chunked form executes at chunk length C (whole
    16x16 tiles): 6 C d_k + 4 C d_v + 6 d_k d_v + C^2/3 with the solve, 2 C (d_k + d_v) +
    4 d_k d_v without. Used for the arithmetic intensity of the attainable roofline."""
    if w.rule in (0, 3):
        return 6 * C * w.dk + 4 * C * w.dv + 6 * w.dk * w.dv + C * C / 3
    return 2 * C * (w.dk + w.dv) + 4 * w.dk * w.dv


def kernel_bytes(w, which):
    """Algorithmic bytes of one launch of each kernel (its own inputs and outputs)."""
    es = 2 if w.dtype == "bf16" else 4
    N = w.B * w.H * w.T
    lam = 0 if w.lam is None else 4 * (w.dk if w.per_channel else 1)
    beta = 0 if w.beta is None else 4
    state = w.B * w.H * w.dk * w.dv * 4
    if w.rule == 3:
        # prep reads q, k, lambda; propagate reads q, k, v and beta [.., d_v]
        if which == "prep":
            return N * (2 * w.dk * es + lam)
        return N * ((2 * w.dk + w.dv) * es + 4 * w.dv + 4 * w.dv) + 2 * state
    if which == "prep":   # reads q, k, beta, lambda
        return N * (2 * w.dk * es + beta + lam)
    # propagate: reads q, k, v (and lambda when per channel), writes out; state in and out
    return N * ((2 * w.dk + w.dv) * es + (lam if w.per_channel else 0) + 4 * w.dv) + 2 * state


def scan_mfma_flops(w, C=64):
    """MFMA flops executed per launch of each kernel (lower-triangular K blocks skipped).

    prep, per (head, chunk): 10 lower 16x16 tiles over K = d_k for each Gram product
    (X X^T for the shifted-pair rules, delta and inner-product, and Q X^T):
    2*16*16*d_k flops per tile.
    propagate, per (head, chunk): X S, Q S and X^T U are 2*C*d_k*d_v each; T R and M U
    take 6 MFMA blocks of 16x16x32 per 16 value columns. The additive and inner-product
    rules have no X S and no T R. Each product is counted once: the split kernels evaluate a product with a
    hi/lo operand as two or three MFMAs, and those repeats are not counted."""
    nch = (w.T + C - 1) // C
    units = w.B * w.H * nch
    if w.rule == 3:
        # G and P (10 lower tiles each); X S, Q S, X^T W~, and the G W~ / P W~ blocks
        # (6 and 10 blocks of 16x16x16 per 16 value columns)
        prep = units * 2 * 10 * 2 * 16 * 16 * w.dk
        blk = 2 * 16 * 16 * 16 * (w.dv // 16)
        return prep, units * (3 * 2 * C * w.dk * w.dv + 16 * blk)
    delta = w.rule == 0
    shifted = w.rule != 1
    tile = 2 * 16 * 16 * w.dk
    prep = units * (2 if shifted else 1) * 10 * tile
    dense = 2 * C * w.dk * w.dv
    tri = 6 * (2 * 16 * 16 * 32) * (w.dv // 16)
    prop = units * ((3 * dense + 2 * tri) if delta else (2 * dense + tri))
    return prep, prop


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="delta_bf16_h16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--backward-steps", type=int, default=3)
    ap.add_argument("--no-copy-calibration", action="store_true",
                    help="skip the plain 1 GiB device copy (the measured-bandwidth reference, "
                         "also the HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the scan shards over heads with no "
              "communication, and the library has no multi-GPU path. Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from linear_attention_scan_amd import fwmem as F
    from linear_attention_scan_amd import workloads as wl

    F.load()  # fails loudly when the library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    w = wl.SCAN_WORKLOADS[args.workload](seed=0)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def dev_t(x, dt=None):
        t = torch.from_numpy(np.ascontiguousarray(x))
        return t.to(dt).to(dev) if dt is not None else t.to(dev)

    q, k, v = dev_t(w.q, tdt), dev_t(w.k, tdt), dev_t(w.v, tdt)
    beta = None if w.beta is None else dev_t(w.beta)
    lam = None if w.lam is None else dev_t(w.lam)
    flags = (F.PHI_ELU1 if w.phi == wl.PHI_ELU1 else 0) | (F.LAMBDA_PER_CHANNEL if w.per_channel else 0)
    if w.qk_norm is not None:
        flags |= {"l2": F.QK_L2NORM, "rms": F.QK_RMSNORM}[w.qk_norm]
    if w.znorm:
        flags |= F.ZNORM
    if w.lam_scaled:
        flags |= F.LAMBDA_SCALED
    shp = F.shape(w.B, w.H, w.T, w.dk, w.dv, F.BF16 if w.dtype == "bf16" else F.F32)
    md = F.mode(w.rule, flags, w.eps, 0)
    out = torch.empty((w.B, w.H, w.T, w.dv), dtype=torch.float32, device=dev)
    S_out = F.State(w.B, w.H, w.dk, w.dv, device=dev)
    ws_n = F.workspace_bytes(shp, md)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)

    def launch(entry):
        st = F.scan_fwd_raw(shp, q, k, v, beta, lam, md, None, out, S_out.buf, ws, ws_n,
                            stream, entry=entry)
        if st != F.OK:
            raise F.FwmemError(st, entry)

    for _ in range(args.warmup):
        launch(F.PHASE_PREP)
        launch(F.PHASE_PROPAGATE)
    torch.cuda.synchronize()

    # Timed region 1, the step rate: K steps back to back, bracketed by synchronisations.
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        launch(F.PHASE_PREP)
        launch(F.PHASE_PROPAGATE)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K

    # Timed region 2, the kernels' launch durations: the same K steps with a HIP event
    # before and after every launch, on the stream the kernels run on. The events add a
    # few microseconds per launch, which is why the step rate is taken without them.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        ev[i][0].record(stream)
        launch(F.PHASE_PREP)
        ev[i][1].record(stream)
        launch(F.PHASE_PROPAGATE)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    ms_prep = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    ms_prop = sum(e[1].elapsed_time(e[2]) for e in ev) / K
    assert bool(torch.isfinite(out).all()), "non-finite output"

    tokens = w.B * w.T
    value = tokens / (ms_step * 1e-3)
    kern = {
        "prep": {"ms": ms_prep, "bytes": kernel_bytes(w, "prep")},
        "propagate": {"ms": ms_prop, "bytes": kernel_bytes(w, "propagate")},
    }
    fl_prep, fl_prop = scan_mfma_flops(w)
    kern["prep"]["mfma_flops"] = fl_prep
    kern["propagate"]["mfma_flops"] = fl_prop
    for name, kk in kern.items():
        kk["GBs"] = kk["bytes"] / (kk["ms"] * 1e-3) / 1e9
        kk["mfma_TFLOPs"] = kk["mfma_flops"] / (kk["ms"] * 1e-3) / 1e12
    dom = max(kern, key=lambda n: kern[n]["ms"])
    names = kernel_names(w)
    copy_gbs = None if args.no_copy_calibration else copy_bandwidth(dev, stream)

    # roofline of the dominant kernel on the algorithmic bytes of the whole scan (q, k, v,
    # o in the input type, the gates), over that kernel's average launch duration
    units = w.B * w.H * w.T
    algo_b = algorithmic_bytes_per_token_head(w) * units
    algo_f = algorithmic_flops_per_token_head(w) * units
    exec_f = executed_flops_per_token_head(w) * units
    dom_s = kern[dom]["ms"] * 1e-3
    step_s = ms_step * 1e-3
    achieved = algo_b / dom_s / 1e9
    # attainable roofline: the longer of the HBM time of the algorithmic bytes and the
    # MFMA time of the executed flops, against the measured time
    t_attain = max(algo_b / (HBM_PEAK_GBS * 1e9), exec_f / (MFMA_BF16_PEAK_TFLOPS * 1e12))
    # the same kernel on the bytes it really moves with the library's float32 output and
    # the state read and written once
    b32 = kern[dom]["bytes"]
    roofline = {
        "bound": "hbm",
        "kernel": names[dom],
        "achieved": round(achieved, 2),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic(w.name, names[dom]),
        "algorithmic_bytes": algo_b,
        "bytes_per_token_head": algorithmic_bytes_per_token_head(w),
        "launch_ms": round(kern[dom]["ms"], 5),
        "whole_step_frac": round(algo_b / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "copy_GBs": copy_gbs,
        "frac_of_copy": None if copy_gbs is None else round(achieved / copy_gbs, 4),
        "attainable_frac": round(t_attain / dom_s, 4),
        "attainable_frac_whole_step": round(t_attain / step_s, 4),
        "algorithmic_flops": algo_f,
        "mfma_TFLOPs": round(algo_f / dom_s / 1e12, 2),
        "mfma_frac": round(algo_f / dom_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "mfma_frac_whole_step": round(algo_f / step_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "fp32_out": {"bytes": b32, "achieved": round(b32 / dom_s / 1e9, 2),
                     "frac": round(b32 / dom_s / 1e9 / HBM_PEAK_GBS, 4)},
    }
    whole_bytes = w.B * w.H * w.T * scan_bytes_per_token_head(w) + 2 * w.B * w.H * w.dk * w.dv * 4

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": compute_dtype(w),
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
                   "rule": ("delta", "additive", "inner", "delta_pv")[w.rule], "inputs": w.dtype,
                   "chunk": 64, "seed": 0, "qk_norm": w.qk_norm, "znorm": w.znorm},
        "roofline": roofline,
        "kernels": {names[n]: {"ms": round(kk["ms"], 5), "GBs": round(kk["GBs"], 1),
                               "mfma_TFLOPs": round(kk["mfma_TFLOPs"], 2),
                               "traffic": measured_traffic(w.name, names[n])}
                    for n, kk in kern.items()},
        "whole_step_GBs": round(whole_bytes / (ms_step * 1e-3) / 1e9, 1),
    }

    if not args.no_decode:
        result["decode"] = bench_decode(args.decode_steps, dev, stream)

    if not args.no_backward and backward_supported(w):
        result["backward"] = bench_backward(w, args.backward_steps, dev, stream, q, k, v, beta, lam)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w)

    print(json.dumps(result), flush=True)


def copy_bandwidth(dev, stream):
    """GB/s of a plain 1 GiB device-to-device copy (bytes read plus bytes written), five
    copies between two HIP events after three untimed ones. Its kernel is also the
    calibration of the HBM counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    gbs = 2 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    return round(gbs, 1)


def backward_supported(w):
    """Whether fwmem_scan_bwd takes the workload's mode: every rule, with the scale-coupled
    ridge only for a scalar lambda and the normaliser only for a scalar decay."""
    return (not (w.lam_scaled and w.per_channel) and not (w.znorm and w.per_channel)
            and w.dk in (64, 128) and w.dv in (64, 128))


def bench_backward(w, steps, dev, stream, q, k, v, beta, lam):
    """fwmem_scan_bwd on the same workload (grad_out ~ N(0,1), zero final-state gradient):
    the time of one call (all its kernels), averaged over `steps` calls bracketed by HIP
    events on the kernels' stream. Algorithmic bytes per (token, head): q, k, v in their input
    type, the gates, grad_out and the float32 gradients of q, k, v and the gates; per head the
    initial-state gradient. `traffic` sums the counter records of the call's kernels while
    every one of them is unchanged."""
    import torch

    from linear_attention_scan_amd import fwmem as F
    from linear_attention_scan_amd import workloads as wl
    shp = F.shape(w.B, w.H, w.T, w.dk, w.dv, F.BF16 if w.dtype == "bf16" else F.F32)
    flags = (F.PHI_ELU1 if w.phi == wl.PHI_ELU1 else 0) | (F.LAMBDA_PER_CHANNEL if w.per_channel else 0)
    if w.qk_norm is not None:
        flags |= {"l2": F.QK_L2NORM, "rms": F.QK_RMSNORM}[w.qk_norm]
    if w.lam_scaled:
        flags |= F.LAMBDA_SCALED
    if w.znorm:
        flags |= F.ZNORM
    md = F.mode(w.rule, flags, w.eps, 0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    gout = torch.randn((w.B, w.H, w.T, w.dv), generator=gen, device=dev)
    gq = torch.empty((w.B, w.H, w.T, w.dk), device=dev)
    gk, gv = torch.empty_like(gq), torch.empty((w.B, w.H, w.T, w.dv), device=dev)
    gb = None if beta is None else torch.empty(tuple(beta.shape), device=dev)
    gl = None if lam is None else torch.empty(tuple(lam.shape), device=dev)
    gS = F.State(w.B, w.H, w.dk, w.dv, device=dev)
    ws_n = F.bwd_workspace_bytes(shp, md)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)

    def one():
        st = F.scan_bwd_raw(shp, q, k, v, beta, lam, md, None, gout, None, gq, gk, gv, gb, gl,
                            gS.buf, ws, ws_n, stream)
        if st != F.OK:
            raise F.FwmemError(st, "fwmem_scan_bwd")

    one()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    evs[0].record(stream)
    for _ in range(steps):
        one()
    evs[1].record(stream)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(gk).all()), "non-finite gradient"
    ms = evs[0].elapsed_time(evs[1]) / steps
    # the chunk-parallel kernels take the scalar-decay delta, inner and additive rules without
    # the normaliser; every other mode runs the token-serial kernel
    chunked = w.rule in (0, 1, 2) and not w.per_channel and not w.znorm
    if chunked and w.dtype == "bf16":  # split operands on bf16 MFMA
        kernels = ["bwd_prep_kernel", "bwd_state_bf_kernel", "bwd_dstate_bf_kernel", "bwd_grad_kernel"]
    elif chunked:  # float32 inputs: float32 MFMA
        kernels = ["bwd_prep_kernel", "bwd_state_kernel", "bwd_dstate_kernel", "bwd_grad_f32_kernel"]
    else:
        kernels = ["bwd_kernel"]
    if w.qk_norm is not None:
        kernels.append("qk_norm_bwd_kernel")
    traffic = None
    if all(measured_traffic(w.name, kname) is not None for kname in kernels):
        traffic = sum(measured_traffic(w.name, kname) for kname in kernels)
    es = 2 if w.dtype == "bf16" else 4
    ngates = ((beta is not None) * (w.dv if w.rule == 3 else 1)
              + (lam is not None) * (w.dk if w.per_channel else 1))
    per_tok = (2 * w.dk + w.dv) * es + 4 * ngates + 4 * w.dv + 4 * (2 * w.dk + w.dv) + 4 * ngates
    nbytes = w.B * w.H * (w.T * per_tok + w.dk * w.dv * 4)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"path": "chunked" if chunked else "token-serial", "kernels": kernels,
            "steps": steps, "ms": round(ms, 4),
            "tokens_per_s": round(w.B * w.T / (ms * 1e-3), 1),
            "workspace_bytes": ws_n,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 5),
                         "traffic": traffic, "bytes_per_launch": nbytes}}


def bench_decode(steps, dev, stream):
    """fwmem_step at B=256, H=32, d=128 (delta rule, lambda = 0.01): HBM stream of the
    512 MiB fp32 state per step, updated in place (S_in == S_out), as a decode loop
    keeps its state. Inputs come from a pool of 16 pre-generated steps."""
    import numpy as np
    import torch

    from linear_attention_scan_amd import fwmem as F
    from linear_attention_scan_amd import workloads as wl
    B, H, d = 256, 32, 128
    pool = []
    for s in range(16):
        inp = wl.decode_step(0, s, B, H, d)
        pool.append(tuple(torch.from_numpy(x).to(dt).to(dev) for x, dt in (
            (inp.q, torch.bfloat16), (inp.k, torch.bfloat16), (inp.v, torch.bfloat16),
            (inp.beta, torch.float32), (inp.lam, torch.float32))))
    sa = F.State(B, H, d, d, device=dev)
    sa.S.copy_(torch.from_numpy(wl.decode_state0(0, B, H, d)))
    out = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    shp = F.shape(B, H, 1, d, d, F.BF16)
    md = F.mode(0, 0, 1e-6, 0)

    def one(i):
        q, k, v, be, la = pool[i % len(pool)]
        st = F.step_raw(shp, q, k, v, be, la, md, sa.buf, out, sa.buf, stream)  # in place
        if st != F.OK:
            raise F.FwmemError(st, "fwmem_step")

    for i in range(20):
        one(i)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    evs[0].record(stream)
    for i in range(steps):
        one(20 + i)
    evs[1].record(stream)
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / steps
    per_head = 2 * d * d * 4 + 3 * d * 2 + 8 + d * 4 + 2 * d * 4 + 8
    nbytes = B * H * per_head
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "decode B=256 H=32 d=128", "kernel": "step_kernel", "steps": steps,
            "state": "in place",
            "ms_per_step": round(ms, 5), "tokens_per_s": round(B / (ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode", "step_kernel"),
                         "bytes_per_launch": nbytes}}


def cpu_baseline(w, min_s=10.0):
    """The fp64 oracle, untuned, on a bounded sample of the same workload: whole batch
    elements (all H heads, all T tokens) in order, repeating the batch if it is done in
    under min_s seconds, until about min_s seconds of CPU work. BLAS is held to one thread,
    so `cores` is exact."""
    from threadpoolctl import threadpool_limits

    from oracle import fwmem_oracle as orc

    def run(b):
        sl = (slice(b, b + 1), slice(None), slice(None))
        # the same computation as the GPU run: the activated gates the library is handed,
        # and every option the workload sets
        orc.scan(w.q[sl], w.k[sl], w.v[sl], None if w.beta is None else w.beta[sl],
                 None if w.lam is None else w.lam[sl], rule=w.rule, phi_kind=w.phi, eps=w.eps,
                 per_channel=w.per_channel, qk_norm=w.qk_norm, znorm=w.znorm,
                 lam_scaled=w.lam_scaled)

    n = 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while True:
            run(n % w.B)
            n += 1
            t = time.perf_counter() - t0
            if t >= min_s:
                break
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(n * w.T / t, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model, "blas_threads": 1,
            "sample": f"{n} batch elements of {w.T} tokens x {w.H} heads (batch elements "
                      f"0..{w.B - 1} in turn), fp64 NumPy recurrence, one thread, {t:.1f} s"}


if __name__ == "__main__":
    main()
