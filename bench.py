"""Benchmark of the deformable convolution forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4] [--all] [--no-cpu]

One step = one full forward (the staging launch, then the fused launch, exactly
what dcn_forward issues) over the workload's synthetic inputs, which are resident
in HBM before timing starts.
The default workload is the ResNet-50 c4 downsampling layer (bf16, B=2,
Cin=Cout=256, 100x168 input, 3x3, stride 2, pad 1 -> 50x84).  Prints one JSON
line; with --all, one line per named workload (the first line is still the
headline workload).

value       = effective TFLOP/s of the whole step, 2*B*Cout*Ho*Wo*Cin*K^2 / step time
              (the timed region has HIP events at its two ends only)
roofline    = the fused kernel alone: algorithmic flops per launch / its mean duration,
              from HIP events recorded around each launch in a second timed pass of K
              steps on the stream the kernels run on, against the dense MFMA peak of the element
              type (HBM peak for the fp32 single-image workload); traffic = HBM bytes
              per launch from the committed counter runs, if the kernels are unchanged
cpu_baseline = the CPU oracle on a bounded slice of the same workload (a range of
              output channels), scaled to TFLOP/s, with the threads it used
clock ramp  = before the W warm-up steps, untimed steps for --ramp-ms of wall time
              (default 200) bring the GPU to its steady clocks
cold        = separate from value: steps each preceded by a 512 MiB device write that
              evicts the inputs from L2 and the 256 MB last-level cache (MALL), timed
              with events around the step alone
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16_mfma": 2516.6, "f32_mfma": 157.3, "hbm": 8000.0}   # TFLOP/s, TFLOP/s, GB/s
CSRC = os.path.join(ROOT, "deformable_convolution_vision_amd", "csrc")
# The library sources each bench workload's launches come from: the host code and the
# staging kernel for every workload, plus the kernels the workload runs.  A change to any
# of them invalidates that workload's committed counter figures.
_COMMON_SRCS = ("dcn_internal.h", "dcn_api.hip", "dcn_kernels.hip")
_BOX_SRCS = ("dcn_box_kernel.h", "dcn_box.hip", "dcn_box_inst_a.hip", "dcn_box_inst_b.hip", "dcn_box_inst_c.hip",
             "dcn_box_inst_d.hip")
_WORKLOAD_SRCS = {
    "c3": _BOX_SRCS, "c4": _BOX_SRCS, "c5": _BOX_SRCS, "c4_g4": _BOX_SRCS,
    "single224": ("dcn_direct.hip",), "tiny": ("dcn_direct.hip",),
    "c4_om": ("dcn_om.hip",), "c4_layer": ("dcn_om.hip",) + _BOX_SRCS,
    "c4_bwd": ("dcn_backward.hip",), "roi_c4": ("dcn_roi.hip",), "psroi_c4": ("dcn_roi.hip",),
}


def _kernel_srcs(workload: str | None = None):
    """The sources behind a workload's launches (every source of the library when the
    workload is not one of the named ones)."""
    if workload in _WORKLOAD_SRCS:
        return tuple(sorted(set(_COMMON_SRCS + _WORKLOAD_SRCS[workload])))
    return tuple(sorted(n for n in os.listdir(CSRC) if n.endswith((".hip", ".h"))))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_hash(workload: str | None = None) -> str:
    """Hash of the sources behind a workload's launches (its counter figures are valid
    only for these)."""
    h = hashlib.sha256()
    for name in _kernel_srcs(workload):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def kernel_symbol(variant: str, plan: str, w) -> str:
    """Device symbol of the fused launch, as rocprofv3 names it."""
    import re
    kk = w.K * w.K
    if variant.startswith("box"):
        m = re.search(r"\((\d+) slots\) x (\d+) ch", plan)
        pw = re.search(r"producer waves=(\d+)", plan)
        grp = re.search(r"offset groups=(\d+)", plan)
        grouped = "true" if grp and int(grp.group(1)) > 1 else "false"
        return (f"dcn_box_kernel<{int(m.group(2)) // 64}, {int(m.group(1)) // 16}, {9 if kk == 9 else 0}, "
                f"{grouped}, {pw.group(1) if pw else 4}>")
    if variant.startswith("direct"):
        bf16 = "true" if variant.endswith("bf16") else "false"
        return f"dcn_direct_kernel<{bf16}, {kk}, {3 if (w.Cin == 3 and kk == 9) else 0}>"
    m = re.match(r"tile_(\w+)_m(\d+)_n(\d+)", variant)
    return f"dcn_fused_kernel<{'true' if m.group(1) == 'bf16' else 'false'}, {m.group(2)}, {m.group(3)}>"


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    """HIP events from the runtime torch has loaded, created without the system-scope
    release fence (a timing marker then adds no cache write-back between launches)."""

    def __init__(self, n: int):
        import ctypes
        path = "libamdhip64.so"
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        self.ct = ctypes
        self.hip = hip = ctypes.CDLL(path)
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)

    def record(self, i: int, stream: int):
        if self.hip.hipEventRecord(self.ev[i], stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def sync(self, i: int):
        if self.hip.hipEventSynchronize(self.ev[i]) != 0:
            raise RuntimeError("hipEventSynchronize failed")

    def ms(self, i: int, j: int) -> float:
        f = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(f), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


def traffic_for(workload: str):
    """HBM bytes per fused launch (per call, all launches, for the offset/mask branch, the
    layer, the backward and RoI pooling) from the committed counter runs, if the sources
    are unchanged."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get(workload)
    if not entry or entry.get("kernel_sha") != kernel_hash(workload):
        return None
    return entry.get("bytes_per_launch")


RAMP_MS = 200.0   # set by --ramp-ms


def clock_ramp(fn) -> float:
    """Untimed calls of fn for RAMP_MS of wall time before the W warm-up steps: the GPU
    reaches its steady clocks only after tens of milliseconds of load, so a short
    warm-up alone (W = 5) would time the clock ramp instead of the kernels.  Returns
    the milliseconds spent."""
    import torch
    if RAMP_MS <= 0:
        return 0.0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < RAMP_MS:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3


def bench_offset_mask(w, steps: int, warmup: int):
    """The DCNv2 offset/mask convolution (dcn_offset_mask): one step is one call (its
    staging launch and its convolution launch), timed as a whole with HIP events."""
    import numpy as np
    import torch

    import deformable_convolution_vision_amd as dcn
    import oracle
    from deformable_convolution_vision_amd.workloads import generate

    host = generate(w)
    g = {k: (None if v is None else v.cuda()) for k, v in host.items()}
    dt = dcn.F32 if w.dtype == "f32" else dcn.BF16
    desc = dcn.make_desc(w.B, w.Cin, w.H, w.W, 1, w.K, w.stride, w.pad, w.dilation, dt, w.groups)
    Ho, Wo = dcn.dcn_output_hw(desc)
    nb = dcn.dcn_offset_mask_workspace_bytes(desc)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    KK = w.K * w.K
    n_off = 2 * w.groups * KK
    off = torch.empty((w.B, n_off, Ho, Wo), dtype=g["x"].dtype, device="cuda")
    msk = torch.empty((w.B, w.groups * KK, Ho, Wo), dtype=g["x"].dtype, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step():
        dcn.dcn_offset_mask(desc, g["x"], g["weight"], g["bias"], off, msk, ws, nb, stream)

    step()
    torch.cuda.synchronize()
    # parity on sampled outputs: the oracle's convolution (zero offsets) at those points
    rng = np.random.default_rng(0)
    npts = 512
    pts = np.stack([rng.integers(0, w.B, npts), rng.integers(0, w.Cout, npts), rng.integers(0, Ho, npts),
                    rng.integers(0, Wo, npts)], 1).astype(np.int64)
    zero = np.zeros((w.B, 2 * KK, Ho, Wo), dtype=np.float32)
    y, a = oracle.points(host["x"], zero, host["weight"], pts, host["bias"], w.stride, w.pad, w.dilation)
    got_off = off.float().cpu().numpy()
    got_msk = msk.float().cpu().numpy()
    tol = 1e-4 if w.dtype == "f32" else 1e-2
    max_rel = 0.0
    for (b, o, oy, ox), yy, aa in zip(pts, y, a):
        if o < n_off:
            err = abs(got_off[b, o, oy, ox] - yy) / max(aa, 1e-30)
        else:   # sigmoid is 1/4-Lipschitz; the mask is rounded to the element type
            ref = 1.0 / (1.0 + np.exp(-yy))
            err = max(abs(got_msk[b, o - n_off, oy, ox] - ref) - (2.0 ** -9 if w.dtype == "bf16" else 1e-6), 0.0) \
                / max(aa / 4, 1e-30)
        max_rel = max(max_rel, float(err))
    if not max_rel <= tol:
        raise SystemExit(f"bench parity failure on {w.name}: max relative error {max_rel:.3e} > {tol}")
    clock_ramp(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = HipEvents(steps + 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(0, sp)
    for i in range(steps):
        step()
        ev.record(i + 1, sp)
    ev.sync(steps)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(ev.ms(i, i + 1) for i in range(steps))
    total_ms = ev.ms(0, steps)
    ev.close()
    ms_per_step = total_ms / steps
    tflops = w.flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK["bf16_mfma"] if w.dtype == "bf16" else PEAK["f32_mfma"]
    gbps = w.algorithmic_bytes / (ms_per_step * 1e-3) / 1e9
    # the kernel dcn_offset_mask runs (its planning rule): bf16 on the convolution kernel
    # of dcn_om.hip, fp32 on the tile kernels
    variant = "om_bf16" if w.dtype == "bf16" else f"tile_f32_m{64 if w.Cout <= 64 else 128}_n64"
    return {
        "metric": "deform_conv2d fwd effective TFLOP/s + GB/s (c4 stride-2 bf16), % of roofline",
        "value": round(tflops, 4), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded; shapes and value distributions of the workload)",
        "config": {"workload": f"{w.name}: offset/mask convolution B={w.B} Cin={w.Cin} {w.H}x{w.W} -> "
                               f"{w.Cout} channels {Ho}x{Wo} (offsets {n_off}, mask {w.groups * KK}), K={w.K} "
                               f"stride={w.stride} pad={w.pad} dilation={w.dilation}",
                   "variant": variant, "plan": "dcn_offset_mask: staging launch + convolution launch"},
        "effective_gbps": round(w.algorithmic_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "frac_mfma_peak": round(tflops / peak, 5),
        "frac_hbm_peak": round(w.algorithmic_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK["hbm"], 5),
        # about 58 flop per algorithmic byte, far below the bf16 ridge: bound by HBM
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": PEAK["hbm"], "unit": "GB/s",
                     "frac": round(gbps / PEAK["hbm"], 5), "traffic": traffic_for(w.name),
                     "kernel": "dcn_offset_mask (both launches)", "kernel_sha": kernel_hash(w.name),
                     "per_launch": {"flops": w.flops, "algorithmic_bytes": w.algorithmic_bytes}},
        "kernels_us": {"call_mean": round(total_ms / steps * 1e3, 3), "call_median": round(per[steps // 2] * 1e3, 3),
                       "call_min": round(per[0] * 1e3, 3)},
        "host_wall_ms_per_step": round(wall * 1e3 / steps, 6),
        "parity_max_rel_err_sampled": max_rel,
        "cold": None,
        "cpu_baseline": None,
    }


def bench_layer(w, steps: int, warmup: int):
    """The whole DCNv2 layer (dcn_layer_forward): the offset/mask branch of the c4 layer
    (256 -> 27 channels) and its deformable convolution (256 -> 256) off one staged copy
    of x, one call per step (staging launch, branch launch, deformable launch).  The same
    work as two separate calls (dcn_offset_mask, then dcn_forward) is timed beside it.
    value is TFLOP/s of both convolutions."""
    import numpy as np
    import torch

    import deformable_convolution_vision_amd as dcn
    import oracle
    from deformable_convolution_vision_amd.workloads import WORKLOADS, generate

    wf, wo = WORKLOADS["c4"], WORKLOADS["c4_om"]
    inp, inp_om = generate(wf), generate(wo)
    inp["x"] = inp_om["x"]
    g = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    go = {k: (None if v is None else v.cuda()) for k, v in inp_om.items()}
    desc = dcn.make_desc(wf.B, wf.Cin, wf.H, wf.W, wf.Cout, wf.K, wf.stride, wf.pad, wf.dilation, dcn.BF16, 1)
    Ho, Wo = dcn.dcn_output_hw(desc)
    nb = dcn.dcn_layer_workspace_bytes(desc)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((wf.B, wf.Cout, Ho, Wo), dtype=torch.bfloat16, device="cuda")
    off = torch.empty((wf.B, 18, Ho, Wo), dtype=torch.bfloat16, device="cuda")
    msk = torch.empty((wf.B, 9, Ho, Wo), dtype=torch.bfloat16, device="cuda")
    nb_om = dcn.dcn_offset_mask_workspace_bytes(desc)
    nb_f = dcn.dcn_workspace_bytes(desc)
    ws_om = torch.empty(max(nb_om, 1), dtype=torch.uint8, device="cuda")
    ws_f = torch.empty(max(nb_f, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step():
        dcn.dcn_layer_forward(desc, g["x"], go["weight"], go["bias"], g["weight"], None, off, msk, out, ws, nb,
                              stream)

    def step_separate():
        dcn.dcn_offset_mask(desc, g["x"], go["weight"], go["bias"], off, msk, ws_om, nb_om, stream)
        dcn.dcn_forward(desc, g["x"], off, msk, g["weight"], None, out, ws_f, nb_f, stream)

    step()
    torch.cuda.synchronize()
    # parity on sampled outputs: the branch against the oracle's convolution, the layer's
    # output against the oracle's forward on the offsets and mask the call produced
    rng = np.random.default_rng(0)
    npts = 512
    pts = np.stack([rng.integers(0, wf.B, npts), rng.integers(0, wf.Cout, npts), rng.integers(0, Ho, npts),
                    rng.integers(0, Wo, npts)], 1).astype(np.int64)
    offh, mskh = off.cpu(), msk.cpu()
    y, a = oracle.points(inp["x"], offh, inp["weight"], pts, None, wf.stride, wf.pad, wf.dilation, mask=mskh)
    got = out.float().cpu().numpy()[pts[:, 0], pts[:, 1], pts[:, 2], pts[:, 3]]
    max_rel = float(np.max(np.abs(got - y) / a))
    pts_o = pts.copy()
    pts_o[:, 1] = rng.integers(0, 27, npts)
    zero = np.zeros((wf.B, 18, Ho, Wo), dtype=np.float32)
    yo, ao = oracle.points(inp["x"], zero, inp_om["weight"], pts_o, inp_om["bias"], wf.stride, wf.pad, wf.dilation)
    for (b, o, oy, ox), yy, aa in zip(pts_o, yo, ao):
        if o < 18:
            e = abs(float(offh[b, o, oy, ox]) - yy) / aa
        else:
            e = max(abs(float(mskh[b, o - 18, oy, ox]) - 1.0 / (1.0 + np.exp(-yy))) - 2.0 ** -9, 0.0) / (aa / 4)
        max_rel = max(max_rel, float(e))
    if not max_rel <= 1e-2:
        raise SystemExit(f"bench parity failure on {w.name}: max relative error {max_rel:.3e} > 1e-2")

    def timed(fn):
        clock_ramp(fn)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = HipEvents(2)
        t0 = time.perf_counter()
        ev.record(0, sp)
        for _ in range(steps):
            fn()
        ev.record(1, sp)
        ev.sync(1)
        wall = time.perf_counter() - t0
        ms = ev.ms(0, 1) / steps
        ev.close()
        return ms, wall

    ms_sep, _ = timed(step_separate)
    ms_per_step, wall = timed(step)
    flops = wf.flops + wo.flops
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK["bf16_mfma"]
    return {
        "metric": "deform_conv2d fwd effective TFLOP/s + GB/s (c4 stride-2 bf16), % of roofline",
        "value": round(tflops, 4), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded; shapes and value distributions of the workload)",
        "config": {"workload": f"{w.name}: the c4 DCNv2 layer in one call: offset/mask convolution 256 -> 27 "
                               f"channels and the deformable convolution 256 -> 256, B=2 100x168 -> 50x84, K=3 "
                               f"stride=2 pad=1, off one staged copy of x",
                   "variant": "layer", "plan": "dcn_layer_forward: staging (x once, both weights) + branch + "
                                               "deformable launch"},
        "separate_calls_ms_per_step": round(ms_sep, 6),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 4), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 5), "traffic": traffic_for(w.name),
                     "kernel": "dcn_layer_forward (all launches)", "kernel_sha": kernel_hash(w.name),
                     "per_launch": {"flops": flops}},
        "kernels_us": {"call_mean": round(ms_per_step * 1e3, 3), "separate_calls_mean": round(ms_sep * 1e3, 3)},
        "host_wall_ms_per_step": round(wall * 1e3 / steps, 6),
        "parity_max_rel_err_sampled": max_rel,
        "cold": None,
        "cpu_baseline": None,
    }


def bench_backward(w, steps: int, warmup: int):
    """The gradients (dcn_backward: every gradient of the layer, one call per step) on the
    layer's shapes with a seeded upstream gradient.  value counts the two gradient
    products (2 x 2*B*Cout*Ho*Wo*Cin*K^2 flops); the timed region has events at its ends
    only, and a second pass with an event after each call gives the call durations."""
    import numpy as np
    import torch

    import deformable_convolution_vision_amd as dcn
    import oracle
    from deformable_convolution_vision_amd.workloads import generate, grad_output

    host = generate(w)
    gy_h = grad_output(w)
    g = {k: (None if v is None else v.cuda()) for k, v in host.items()}
    gy = gy_h.cuda()
    desc = dcn.describe(g["x"], g["weight"], w.stride, w.pad, w.dilation, g["offset"])
    nb = dcn.dcn_backward_workspace_bytes(desc)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(g["x"]), torch.empty_like(g["offset"]),
            torch.empty_like(g["mask"]) if g["mask"] is not None else None, torch.empty_like(g["weight"]),
            torch.empty(w.Cout, dtype=g["x"].dtype, device="cuda")]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step():
        dcn.dcn_backward(desc, g["x"], g["offset"], g["mask"], g["weight"], gy, *outs, ws, nb, stream)

    step()
    torch.cuda.synchronize()
    # parity on slices the oracle computes in seconds: the weight and bias gradients of
    # the first and last output channels (they depend on those channels of grad_out
    # only) and the input gradient of the first and last input channels (one offset
    # group: they depend on those channels of x and weight only)
    rtol, atol = (1e-2, 2e-3) if w.dtype == "bf16" else (1e-4, 1e-5)
    max_rel = 0.0
    osel = [0, w.Cout - 1]
    ref = oracle.backward(host["x"], host["offset"], host["weight"][osel].contiguous(), gy_h[:, osel].contiguous(),
                          w.stride, w.pad, w.dilation, mask=host["mask"], want=("grad_weight", "grad_bias"))
    csel = [0, w.Cin - 1]
    refx = oracle.backward(host["x"][:, csel].contiguous(), host["offset"], host["weight"][:, csel].contiguous(),
                           gy_h, w.stride, w.pad, w.dilation, mask=host["mask"], want=("grad_x",))
    for got, want in ((outs[3][osel], ref["grad_weight"]), (outs[4][osel], ref["grad_bias"]),
                      (outs[0][:, csel], refx["grad_x"])):
        got = got.float().cpu().numpy().astype(np.float64)
        bound = rtol * np.abs(want) + atol * float(np.max(np.abs(want)))
        max_rel = max(max_rel, float(np.max(np.abs(got - want) / np.maximum(bound, 1e-300))) * rtol)
        if not np.all(np.abs(got - want) <= bound):
            raise SystemExit(f"bench parity failure on {w.name}: gradient outside |d| <= {rtol}|ref| + {atol}max|ref|")
    clock_ramp(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = HipEvents(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(0, sp)
    for _ in range(steps):
        step()
    ev.record(1, sp)
    ev.sync(1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = ev.ms(0, 1)
    ev.close()
    ev = HipEvents(steps + 1)
    ev.record(0, sp)
    for i in range(steps):
        step()
        ev.record(i + 1, sp)
    ev.sync(steps)
    per = sorted(ev.ms(i, i + 1) for i in range(steps))
    call_mean = ev.ms(0, steps) / steps
    ev.close()
    ms_per_step = total_ms / steps
    flops = 2 * w.flops
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK["bf16_mfma"] if w.dtype == "bf16" else PEAK["f32_mfma"]
    achieved = flops / (call_mean * 1e-3) / 1e12
    return {
        "metric": "deform_conv2d fwd effective TFLOP/s + GB/s (c4 stride-2 bf16), % of roofline",
        "value": round(tflops, 4), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded; shapes and value distributions of the workload)",
        "config": {"workload": f"{w.name}: gradients of B={w.B} Cin={w.Cin} {w.H}x{w.W} -> Cout={w.Cout} "
                               f"{w.Ho}x{w.Wo}, K={w.K} stride={w.stride} pad={w.pad} dilation={w.dilation}, "
                               f"mask={'yes' if w.mask else 'no'} (grad x, offset, mask, weight, bias)",
                   "variant": "backward", "plan": "dcn_backward: channels-last staging, transposes, pair count "
                                                   "and scan, column-gradient MFMA product, sampling, input-gradient "
                                                   "gather, weight-gradient MFMA product and split sum"},
        "frac_mfma_peak": round(tflops / peak, 5),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 4), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 5), "traffic": traffic_for(w.name),
                     "kernel": "dcn_backward (all launches of one call)", "kernel_sha": kernel_hash(w.name),
                     "per_launch": {"flops": flops}},
        "kernels_us": {"call_mean": round(call_mean * 1e3, 3), "call_median": round(per[steps // 2] * 1e3, 3),
                       "call_min": round(per[0] * 1e3, 3)},
        "host_wall_ms_per_step": round(wall * 1e3 / steps, 6),
        "parity_max_rel_err_sampled": max_rel,
        "cold": None,
        "cpu_baseline": None,
    }


def bench_roi(w, steps: int, warmup: int):
    """Deformable RoI pooling (dcn_roi_pool), or its position-sensitive form
    (dcn_ps_roi_pool), on the workload's feature map: 256 RoIs per image of an 800 x 1344
    image at spatial scale 1/16, k x k bins (k = the workload's K), 2 x 2 samples per bin,
    per-bin offsets and mask.  One step is one call (plain bf16 pooling: the channels-last
    staging launch and the pooling launch; position-sensitive: one launch).  value is the
    effective bandwidth of its algorithmic bytes (x, rois, offsets and mask read once, the
    output written once); the timed region has events at its ends only."""
    import numpy as np
    import torch

    import deformable_convolution_vision_amd as dcn
    import oracle
    from deformable_convolution_vision_amd.workloads import roi_inputs

    ps = w.op == "ps_roi_pool"
    k, S, scale, gamma, per_img = w.K, 2, 1.0 / 16, 0.1, 256
    host = roi_inputs(w, per_img, k, (800, 1344))
    g = {key: v.cuda() for key, v in host.items()}
    R = g["rois"].shape[0]
    C_out = w.Cout if ps else w.Cin
    dt = dcn.BF16 if w.dtype == "bf16" else dcn.F32
    out = torch.empty((R, C_out, k, k), dtype=g["x"].dtype, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    if ps:
        desc = dcn.PsRoiDesc(w.B, C_out, w.H, w.W, R, k, S, 1, scale, gamma, dt, 0)
        nb = dcn.dcn_ps_roi_pool_workspace_bytes(desc)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")

        def step():
            dcn.dcn_ps_roi_pool(desc, g["x"], g["rois"], g["offset"], g["mask"], out, ws if nb else None, nb, stream)
    else:
        desc = dcn.RoiDesc(w.B, w.Cin, w.H, w.W, R, k, S, scale, gamma, dt, 0)
        nb = dcn.dcn_roi_pool_workspace_bytes(desc)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")

        def step():
            dcn.dcn_roi_pool(desc, g["x"], g["rois"], g["offset"], g["mask"], out, ws if nb else None, nb, stream)

    step()
    torch.cuda.synchronize()
    pool = oracle.ps_roi_pool if ps else oracle.roi_pool
    ref, ab = pool(host["x"], host["rois"], k, S, scale, gamma, host["offset"], host["mask"], with_abs=True)
    tol = 1e-2 if w.dtype == "bf16" else 1e-4
    err = np.abs(out.float().cpu().numpy().astype(np.float64) - ref)
    if np.any(err[ab == 0] != 0):
        raise SystemExit(f"bench parity failure on {w.name}: an output with no terms is not exact")
    max_rel = float(np.max(err[ab > 0] / ab[ab > 0]))
    if not max_rel <= tol:
        raise SystemExit(f"bench parity failure on {w.name}: max relative error {max_rel:.3e} > {tol}")
    clock_ramp(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = HipEvents(2)
    t0 = time.perf_counter()
    ev.record(0, sp)
    for _ in range(steps):
        step()
    ev.record(1, sp)
    ev.sync(1)
    wall = time.perf_counter() - t0
    total_ms = ev.ms(0, 1)
    ev.close()
    ms_per_step = total_ms / steps
    es = 2 if w.dtype == "bf16" else 4
    abytes = es * (w.B * w.Cin * w.H * w.W + R * 2 * k * k + R * k * k + R * C_out * k * k) + 4 * 5 * R
    gbps = abytes / (ms_per_step * 1e-3) / 1e9
    if ps:
        what = (f"{w.name}: deformable position-sensitive RoI pooling of {w.Cin} score maps ({C_out} classes x "
                f"{k}x{k} bins) [{w.B},{w.Cin},{w.H},{w.W}], {R} RoIs ({per_img} per image, sides 32-512 px of "
                f"800x1344, scale 1/16), {S}x{S} samples, one offset per bin, mask")
        plan, kname = ("dcn_ps_roi_pool: staging launch (score maps channels-last, bin-major) + pooling launch",
                       "roi_pool_cl_kernel (position-sensitive)")
    else:
        what = (f"{w.name}: deformable RoI pooling of x [{w.B},{w.Cin},{w.H},{w.W}], {R} RoIs ({per_img} per image, "
                f"sides 32-512 px of 800x1344, scale 1/16), {k}x{k} bins, {S}x{S} samples, offsets and mask")
        plan, kname = "dcn_roi_pool: channels-last staging launch + pooling launch", "roi_pool_cl_kernel"
    return {
        "metric": "deform_conv2d fwd effective TFLOP/s + GB/s (c4 stride-2 bf16), % of roofline",
        "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded; shapes and value distributions of the workload)",
        "config": {"workload": what, "variant": w.op, "plan": plan},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 2), "peak": PEAK["hbm"], "unit": "GB/s",
                     "frac": round(gbps / PEAK["hbm"], 5), "traffic": traffic_for(w.name),
                     "kernel": kname, "kernel_sha": kernel_hash(w.name),
                     "per_launch": {"algorithmic_bytes": abytes, "outputs": R * C_out * k * k}},
        "kernels_us": {"call_mean": round(ms_per_step * 1e3, 3)},
        "host_wall_ms_per_step": round(wall * 1e3 / steps, 6),
        "parity_max_rel_err_sampled": max_rel,
        "cold": None,
        "cpu_baseline": None,
    }


def bench_workload(name: str, steps: int, warmup: int, cpu: bool, cpu_seconds: float, cold_steps: int = 0):
    import numpy as np
    import torch

    import deformable_convolution_vision_amd as dcn
    from deformable_convolution_vision_amd.workloads import WORKLOADS, generate

    w = WORKLOADS[name]
    if w.op == "offset_mask":
        return bench_offset_mask(w, steps, warmup)
    if w.op == "backward":
        return bench_backward(w, steps, warmup)
    if w.op == "layer":
        return bench_layer(w, steps, warmup)
    if w.op in ("roi_pool", "ps_roi_pool"):
        return bench_roi(w, steps, warmup)
    host = generate(w)
    g = {k: (None if v is None else v.cuda()) for k, v in host.items()}
    desc = dcn.describe(g["x"], g["weight"], w.stride, w.pad, w.dilation, g["offset"])
    Ho, Wo = dcn.check_tensors(desc, g["x"], g["offset"], g["weight"], g["bias"], g["mask"])
    assert (Ho, Wo) == (w.Ho, w.Wo)
    nb = dcn.dcn_workspace_bytes(desc)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.B, w.Cout, Ho, Wo), dtype=g["x"].dtype, device="cuda")
    variant = dcn.dcn_variant_name(desc)
    plan = dcn.dcn_plan_describe(desc)
    stream = torch.cuda.current_stream()
    wsp = ws if nb else None

    def step():
        dcn.dcn_forward(desc, g["x"], g["offset"], g["mask"], g["weight"], g["bias"], out, wsp, nb, stream)

    # parity on sampled outputs before timing (same launch configuration)
    step()
    torch.cuda.synchronize()
    import oracle
    rng = np.random.default_rng(0)
    npts = 512
    pts = np.stack([rng.integers(0, w.B, npts), rng.integers(0, w.Cout, npts), rng.integers(0, Ho, npts),
                    rng.integers(0, Wo, npts)], 1).astype(np.int64)
    y, a = oracle.points(host["x"], host["offset"], host["weight"], pts, host["bias"], w.stride, w.pad,
                         w.dilation, mask=host["mask"])
    got = out.float().cpu().numpy()[pts[:, 0], pts[:, 1], pts[:, 2], pts[:, 3]]
    tol = 1e-4 if w.dtype == "f32" else 1e-2
    rel = np.where(a > 0, np.abs(got - y) / np.where(a > 0, a, 1), np.abs(got - y))
    max_rel = float(rel.max())
    if not max_rel <= tol:
        raise SystemExit(f"bench parity failure on {name}: max relative error {max_rel:.3e} > {tol}")

    clock_ramp(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K steps back to back (dcn_forward: the staging launch, then the
    # fused launch), with HIP events only at its two ends.
    sp = stream.cuda_stream
    ev = HipEvents(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(0, sp)
    for _ in range(steps):
        step()
    ev.record(1, sp)
    ev.sync(1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = ev.ms(0, 1)
    ev.close()
    ms_per_step = total_ms / steps

    # Kernel durations: K more steps, timed the same way, with an event recorded between
    # the two launches of each step as well (on the stream they run on), so each
    # kernel's duration is read from its own pair of events.  These events are kept out
    # of the first region: each adds about a microsecond to the step.
    ev = HipEvents(2 * steps + 1)
    torch.cuda.synchronize()
    ev.record(0, sp)
    for i in range(steps):
        dcn.dcn_stage(desc, g["x"], g["weight"], wsp, nb, stream)
        ev.record(2 * i + 1, sp)
        dcn.dcn_forward_staged(desc, g["x"], g["offset"], g["mask"], g["weight"], g["bias"], out, wsp, nb,
                               stream)
        ev.record(2 * i + 2, sp)
    ev.sync(2 * steps)
    torch.cuda.synchronize()
    instr_ms_per_step = ev.ms(0, 2 * steps) / steps
    stage_ms = sorted(ev.ms(2 * i, 2 * i + 1) for i in range(steps))
    fused_ms = sorted(ev.ms(2 * i + 1, 2 * i + 2) for i in range(steps))
    ev.close()
    fused_mean = sum(fused_ms) / steps
    stage_mean = sum(stage_ms) / steps

    cold = None
    if cold_steps > 0:
        # Cold caches: before each step, write 512 MiB (twice the MALL) so that no input
        # byte is left in L2 or the MALL; only the step itself is between the events.
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cev = HipEvents(3 * cold_steps)
        for i in range(cold_steps):
            flush.fill_(i & 0xff)
            cev.record(3 * i, sp)
            dcn.dcn_stage(desc, g["x"], g["weight"], wsp, nb, stream)
            cev.record(3 * i + 1, sp)
            dcn.dcn_forward_staged(desc, g["x"], g["offset"], g["mask"], g["weight"], g["bias"], out, wsp, nb,
                                   stream)
            cev.record(3 * i + 2, sp)
        cev.sync(3 * cold_steps - 1)
        torch.cuda.synchronize()
        c_step = [cev.ms(3 * i, 3 * i + 2) for i in range(cold_steps)]
        c_stage = [cev.ms(3 * i, 3 * i + 1) for i in range(cold_steps)]
        c_fused = [cev.ms(3 * i + 1, 3 * i + 2) for i in range(cold_steps)]
        cev.close()
        del flush
        c_ms = sum(c_step) / cold_steps
        cold = {"steps": cold_steps, "ms_per_step": round(c_ms, 6),
                "tflops": round(w.flops / (c_ms * 1e-3) / 1e12, 4),
                "stage_mean_us": round(sum(c_stage) / cold_steps * 1e3, 3),
                "fused_mean_us": round(sum(c_fused) / cold_steps * 1e3, 3)}

    flops = w.flops
    abytes = w.algorithmic_bytes
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    gbps = abytes / (ms_per_step * 1e-3) / 1e9
    if w.name == "single224":
        bound, peak, unit = "hbm", PEAK["hbm"], "GB/s"
        achieved = abytes / (fused_mean * 1e-3) / 1e9
    else:
        bound, unit = "mfma", "TFLOP/s"
        peak = PEAK["bf16_mfma"] if w.dtype == "bf16" else PEAK["f32_mfma"]
        achieved = flops / (fused_mean * 1e-3) / 1e12
    traffic = traffic_for(name)

    rec = {
        "metric": "deform_conv2d fwd effective TFLOP/s + GB/s (c4 stride-2 bf16), % of roofline",
        "value": round(tflops, 4),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; shapes and value distributions of the workload)",
        "config": {"workload": f"{w.name}: B={w.B} Cin={w.Cin} {w.H}x{w.W} -> Cout={w.Cout} {Ho}x{Wo}, "
                               f"K={w.K} stride={w.stride} pad={w.pad} dilation={w.dilation}, "
                               f"mask={'yes' if w.mask else 'no'}, bias={'yes' if w.bias else 'no'}"
                               + (f", offset groups={w.groups}" if w.groups > 1 else ""),
                   "variant": variant, "plan": plan},
        "effective_gbps": round(gbps, 2),
        "frac_mfma_peak": round(tflops / (PEAK["bf16_mfma"] if w.dtype == "bf16" else PEAK["f32_mfma"]), 5),
        "frac_hbm_peak": round(gbps / PEAK["hbm"], 5),
        "roofline": {"bound": bound, "achieved": round(achieved, 4), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 5), "traffic": traffic,
                     "kernel": kernel_symbol(variant, plan, w), "kernel_sha": kernel_hash(name),
                     "per_launch": {"flops": flops, "algorithmic_bytes": abytes}},
        "kernels_us": {"stage_mean": round(stage_mean * 1e3, 3), "fused_mean": round(fused_mean * 1e3, 3),
                       "fused_median": round(fused_ms[steps // 2] * 1e3, 3),
                       "fused_min": round(fused_ms[0] * 1e3, 3),
                       "instrumented_ms_per_step": round(instr_ms_per_step, 6)},
        "host_wall_ms_per_step": round(wall * 1e3 / steps, 6),
        "parity_max_rel_err_sampled": max_rel,
        "cold": cold,
        "clock_ramp_ms": RAMP_MS,
        "cpu_baseline": None,
    }
    if cpu:
        rec["cpu_baseline"] = cpu_baseline(w, host, cpu_seconds)
    return rec


def cpu_baseline(w, host, target_s: float):
    """The oracle as it stands on a bounded slice (a range of output channels)."""
    import oracle
    kw = dict(mask=host["mask"], with_abs=False)
    args = (host["x"], host["offset"], host["weight"], host["bias"], w.stride, w.pad, w.dilation)
    n1 = max(1, min(w.Cout, 4))
    oracle.forward(*args, cout_range=(0, 1), **kw)          # first-touch warm-up
    t = time.perf_counter()
    oracle.forward(*args, cout_range=(0, n1), **kw)
    t1 = time.perf_counter() - t
    n = int(min(w.Cout, max(n1, round(target_s / max(t1, 1e-6) * n1))))
    t = time.perf_counter()
    oracle.forward(*args, cout_range=(0, n), **kw)
    dt = time.perf_counter() - t
    flops = 2 * w.B * n * w.Ho * w.Wo * w.Cin * w.K * w.K
    return {"value": round(flops / dt / 1e12, 8), "unit": "TFLOP/s", "cores": oracle.threads_used(),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"output channels [0,{n}) of {w.Cout} ({n / w.Cout:.1%} of the workload), all pixels, "
                      f"all batches; fp64 accumulate",
            "affinity_cores": len(os.sched_getaffinity(0))}


def copy_calibration(nbytes: int, reps: int) -> int:
    """A plain copy of known size, so HBM counters can be scaled to bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_bytes": nbytes, "reps": reps, "ms_per_copy": round(ms, 5),
                      "gbps_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # ~0.1 s of back-to-back steps: the GPU reaches its steady clocks only after tens of
    # milliseconds of load (c4 fused launch: 35.1 us after 20 warm-up steps, 33.1 us
    # after 2000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--ramp-ms", type=float, default=200.0,
                    help="untimed steps for this many ms before the warm-up steps (steady GPU clocks)")
    ap.add_argument("--workload", default="c4")
    ap.add_argument("--all", action="store_true", help="also print one line per other named workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="steps timed after evicting the caches (reported under 'cold'; 0 skips them)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device-to-device copy of this many bytes (counter calibration)")
    args = ap.parse_args(argv)
    global RAMP_MS
    RAMP_MS = args.ramp_ms
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (this build has no "
              f"multi-GPU path: the forward shards by batch or output channel with no exchange).",
              file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_bytes:
        return copy_calibration(args.copy_bytes, max(args.steps, 1))
    names = [args.workload]
    if args.all:
        from deformable_convolution_vision_amd.workloads import ORDER
        names += [n for n in ORDER if n != args.workload]
    for i, n in enumerate(names):
        rec = bench_workload(n, args.steps, args.warmup, cpu=(not args.no_cpu) and i == 0,
                             cpu_seconds=args.cpu_seconds, cold_steps=args.cold_steps)
        print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
