"""Benchmark of the four-direction GSPN line-scan forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload profile]

A step is one gspn_forward4 call (normalise the logits, scan T->B, B->T,
L->R, R->L, merge by summation, or with --merge by seeded learnable weights
per direction and channel) over one batch of seeded synthetic inputs already
resident in HBM; for the proxy workload a step is the compressive proxy
pipeline (1x1 projection down, forward4 in proxy space, 1x1 projection up).
--pass backward times gspn_backward4 instead (gspn_proxy_backward4 for the
proxy workload); --pass train a training step, the forward keeping its states
and the backward reading them.  Prints one JSON line.

Measurements:
  - ms per step: HIP events on the stream the library launches on, bracketing
    the K timed steps (synchronised on both sides).
  - stage times: the same call through its *_timed entry point, which records
    HIP events on that stream around every launch of the step.  The dominant
    kernel is the line scan; its per-launch duration is the scan stage's time
    divided by its launch count.
  - roofline.achieved: the algorithmic bytes of the units the dominant
    launch processes (the step's compulsory bytes: every distinct input of
    the four-direction scan read once and its output written once, divided
    over the launches that share the scan) / its per-launch duration;
    roofline.frac = achieved / 8 TB/s.  roofline.design_bytes_per_launch and
    design_achieved give the bytes the launch's design moves (e.g. x and its
    transpose, four partial maps) for comparison.
  - roofline.traffic: HBM bytes per scan launch measured with the FETCH_SIZE
    and WRITE_SIZE counters, read from the committed counter summary under
    profiles/ when it was taken on the current kernel sources, else null;
    step_traffic: the same counters summed over every kernel of the step
    (profiles/step_<workload>_traffic.txt), else null.
  - effective bandwidth of the whole step: algorithmic bytes of the forward
    (every distinct input read once, y written once) / ms per step.
  - cpu_baseline: the fp64 oracle on a bounded sample of the same workload,
    on the host's cores (N = 1 only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from linear_spatial_propagation_gspn_amd import gspn as G  # noqa: E402
from linear_spatial_propagation_gspn_amd.workloads import WORKLOADS, make_inputs  # noqa: E402

HBM_PEAK_GBPS = 8000.0
METRIC = "ms per 4-direction GSPN forward at 1024², B=16, C=8; achieved HBM GB/s"
CSRC = os.path.join(ROOT, "linear_spatial_propagation_gspn_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def esize(wl) -> int:
    return 4 if wl.dtype == "f32" else 2


def unit_bytes(wl) -> int:
    """U: one map of the scanned tensor (n * c_scan * h * w elements)."""
    return wl.n * wl.c_scan * wl.h * wl.w * esize(wl)


def prenormalised(wl) -> bool:
    """Channel-shared logits over several channels are normalised once into
    fp32 weights that the scans read."""
    return wl.cw == 1 and wl.c_scan > 1


def weight_bytes_per_direction(wl) -> int:
    """Bytes of one direction's weights as the scan reads them: the logits
    (three per position and channel), or for prenormalised weights fp32
    triples (fp32 storage) or packed half pairs, 4 bytes a position (bf16)."""
    if prenormalised(wl):
        return wl.n * wl.h * wl.w * (3 * 4 if wl.dtype == "f32" else 4)
    return wl.n * wl.cw * 3 * wl.h * wl.w * esize(wl)


def algorithmic_bytes(wl) -> int:
    """Every distinct input of the step read once and y written once."""
    es = esize(wl)
    hw = wl.h * wl.w
    x = wl.n * wl.c * hw * es
    lam = 4 * wl.n * wl.c_scan * hw * es
    z = 4 * wl.n * wl.cw * 3 * hw * es
    wts = 2 * wl.c * wl.c_proxy * es if wl.c_proxy else 0
    return x + lam + z + wts + x


def scan_algorithmic_bytes(wl) -> int:
    """Compulsory bytes of the four-direction scan of the scanned tensor (in
    proxy space for proxy workloads): x read once, the four directions'
    logits and lambdas read once as stored, y written once: 18U for fp32
    per-channel logits, 6U + 12 N H W 2 bytes for bf16 shared logits."""
    u = unit_bytes(wl)
    z = 4 * wl.n * wl.cw * 3 * wl.h * wl.w * esize(wl)
    return u + 4 * u + z + u


def seq4_launch_planes(wl, cus: int, tail_ran: bool) -> int:
    """The planes the plane-sequential launch processes: all n * c, or,
    when the library ran the last, at most half-full round of one plane per
    CU on the concurrent path (the "tail" stage), all but those."""
    planes = wl.n * wl.c_scan
    return planes - planes % cus if tail_ran and cus > 0 else planes


def projection_bytes(wl, down: bool) -> int:
    """Compulsory bytes of one 1x1 projection of the proxy pipeline: the
    input read once, the output written once, the weights read once (down:
    C -> C_proxy, up: C_proxy -> C)."""
    es = esize(wl)
    hw = wl.h * wl.w
    return wl.n * (wl.c + wl.c_proxy) * hw * es + wl.c * wl.c_proxy * es


# The projection kernels the proxy workload runs (bf16 MFMA paths).
PROJECTION_KERNELS = {"project_down": "project_narrow_out_mfma", "project_up": "project_narrow_in_mfma"}


def launch_algorithmic_bytes(wl, launches: int) -> int:
    """The algorithmic bytes of the units one scan launch processes: the
    scan's compulsory bytes divided over the launches that carry it (one
    fused launch; a band of steps each; one direction each)."""
    return scan_algorithmic_bytes(wl) // max(1, launches)


def scan_launch_bytes(wl, kernel: str, launches: int = 1) -> int:
    """Algorithmic bytes of one launch of the scan kernel the step ran: every
    tensor the launch reads or writes, moved once.
      plane4_kernel (one launch, planes in LDS): x, the four directions'
        logits and lambdas, y written;
      scan4v_kernel / scan4lp_kernel (one launch): x and its transpose, four
        directions' weights and lambdas, four output maps written;
      scan4band_kernel (one launch per band of steps): the long-line
        kernel's bytes spread over the bands (the band-boundary states, a few
        MB, are not counted);
      seq4_kernel (one launch, the planes in turn): x four times, the
        lambdas and weights once, the scratch map z 4U, y 3U;
      scan_kernel (one launch per direction): x (or its transpose), the
        direction's weights and lambda, the output written, and read as well
        by the two launches that add into a map (average over the four)."""
    u = unit_bytes(wl)
    if kernel == "plane4_kernel":
        return u + 4 * wl.n * wl.cw * 3 * wl.h * wl.w * esize(wl) + 4 * u + u
    wd = weight_bytes_per_direction(wl)
    if kernel == "seq4_kernel":
        # x read in each of the four phases, each lambda and weight stream
        # once, the transposed scratch z written, read and written, read
        # (4U), y written, read and written (3U)
        return 4 * u + 4 * u + 4 * wd + 4 * u + 3 * u
    if kernel in ("scan4v_kernel", "scan4lp_kernel"):
        return 2 * u + 4 * wd + 4 * u + 4 * u
    if kernel == "scan4band_kernel":
        return (2 * u + 4 * wd + 4 * u + 4 * u) // launches
    total = 4 * u + 4 * wd + 4 * u + 4 * u + 2 * u
    return total // 4


def backward_algorithmic_bytes(wl) -> int:
    """Backward: x, dL/dy, the logits and lambdas read once; dx, dlambda and
    dlogits written once."""
    u = unit_bytes(wl)
    z = 4 * wl.n * wl.cw * 3 * wl.h * wl.w * esize(wl)
    return 2 * u + z + 4 * u + u + 4 * u + z


def proxy_backward_bytes(wl) -> int:
    """Compulsory bytes of the compressive-proxy backward: x and dL/dy read
    and dx written (C channels); in proxy space the logits and lambdas read
    and their gradients written; both projection weights read and their fp32
    gradients written."""
    es = esize(wl)
    hw = wl.h * wl.w
    big = wl.n * wl.c * hw * es
    lam = 4 * wl.n * wl.c_proxy * hw * es
    z = 4 * wl.n * wl.cw * 3 * hw * es
    return 3 * big + 2 * lam + 2 * z + 2 * wl.c * wl.c_proxy * es + 2 * wl.c * wl.c_proxy * 4


def wgrad_pass_bytes(wl) -> int:
    """Compulsory bytes of one weight-gradient pass of the proxy backward,
    the average of the two: over dL/dy (C channels) and y_p read, dL/dy_p
    written; over x (C channels) and dx_p read."""
    hw = wl.h * wl.w
    big = wl.n * wl.c * hw * esize(wl)
    small = wl.n * wl.c_proxy * hw * esize(wl)
    return (2 * big + 3 * small) // 2


def adjoint_launch_bytes(wl) -> int:
    """Algorithmic bytes of the adjoint launch: x and dL/dy in both frames,
    four lambdas and logits, four fp32 state maps read; four dlambda and dx
    terms written; the logit gradients written (per-channel) or, for shared
    logits, two fp32 sums a position (weight-gradient differences) added into."""
    u = unit_bytes(wl)
    z = 4 * wl.n * wl.cw * 3 * wl.h * wl.w * esize(wl)
    states = 4 * wl.n * wl.c_scan * wl.h * wl.w * 4
    dz = 4 * wl.n * 2 * wl.h * wl.w * 4 if prenormalised(wl) else z  # shared: two fp32 sums a position
    return 2 * u + 2 * u + 4 * u + z + states + 4 * u + 4 * u + dz


def adjplane_launch_bytes(wl) -> int:
    """Algorithmic bytes of the plane-resident adjoint launch (planes of at
    most 64 x 64), which recomputes the forward states itself: x and dL/dy,
    four lambdas and logits read once; four dlambda, the logit gradients
    (per-channel) or their fp32 sums (shared) and dx written once.  The fp32
    states it writes and reads back are its own scratch, not counted (the
    counters show what they cost)."""
    u = unit_bytes(wl)
    z = 4 * wl.n * wl.cw * 3 * wl.h * wl.w * esize(wl)
    dz = 4 * wl.n * 2 * wl.h * wl.w * 4 if prenormalised(wl) else z  # shared: two fp32 sums a position
    return 2 * u + 4 * u + z + 4 * u + dz + u


def merge_weights(wl, on: bool):
    """Seeded learnable merge weights [4][C] (C of the scanned tensor), or None."""
    if not on:
        return None
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed + 2000)
    return torch.randn((4, wl.c_scan), generator=g, device="cuda", dtype=torch.float32)


def array_layout(inp: dict) -> dict:
    """The inputs with every direction's logits and lambda in the array frame
    [.., H, W] (the horizontal directions' transposed; the vertical ones are
    the same tensors)."""
    out = dict(inp)
    for key in ("logits", "lam"):
        out[key] = [t if d < 2 else t.transpose(-1, -2).contiguous() for d, t in enumerate(inp[key])]
    return out


def run_step(wl, inp, out, ws, timed=False, merge=None, layout="scan"):
    if wl.c_proxy:
        f = G.gspn_proxy_forward4_timed if timed else G.gspn_proxy_forward4
        return f(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"],
                 chunk_len=wl.chunk, out=out, workspace=ws, merge=merge, layout=layout)
    f = G.gspn_forward4_timed if timed else G.gspn_forward4
    return f(inp["x"], inp["logits"], inp["lam"], chunk_len=wl.chunk, out=out, workspace=ws, merge=merge,
             layout=layout)


def stage_times(wl, inp, out, ws, reps: int, merge=None, layout="scan") -> dict:
    """Mean per-step duration and launch count of each stage over reps timed
    steps."""
    acc = {name: {"ms": 0.0, "launches": 0} for name in G.STAGES}
    kernel = None
    for _ in range(reps):
        _, t = run_step(wl, inp, out, ws, timed=True, merge=merge, layout=layout)
        kernel = t.pop("scan_kernel")
        t.pop("adjoint_plan")
        for name, v in t.items():
            acc[name]["ms"] += v["ms"] / reps
            acc[name]["launches"] = v["launches"]
    return acc, kernel


# The sources each measured kernel is built from: its own file, the headers
# its device code includes, the launch code that configures it (in the same
# files) and the build flags.  launch.hpp only declares host launchers.
_SCAN4 = ["scan_kernel.hpp", "scan_lp.hpp", "coltile.hpp", "scan.hip", "scan4_f32.hip", "scan4_f32x.hip",
          "scan4_bf16.hip", "scan4_bf16pair.hip"]
KERNEL_SOURCES = {
    "scan4lp_kernel": _SCAN4,
    "scan4band_kernel": _SCAN4 + ["scan_band.hpp"],
    "scan4v_kernel": _SCAN4,
    "plane4_kernel": ["plane4.hip", "plane_common.hpp"],
    "adj4_kernel": ["backward.hip"],
    "adj4band_kernel": ["backward.hip"],
    "adjplane_kernel": ["adjplane.hip", "plane_common.hpp"],
    "seq4_kernel": ["seq4.hip", "coltile.hpp"],
    "project_narrow_out_mfma": ["project.hip"],
    "project_narrow_in_mfma": ["project.hip"],
    "wgrad_mfma": ["wgrad.hip"],
}
_COMMON = ["device.hpp", "check.hpp"]


def kernel_sources_digest(kernel: str | None = None) -> str:
    """sha256 over the sources of one kernel (KERNEL_SOURCES, plus the shared
    device helpers and build.py), or over every kernel source of the library
    for an unlisted kernel."""
    if kernel in KERNEL_SOURCES:
        names = sorted(set(KERNEL_SOURCES[kernel] + _COMMON))
    else:
        names = sorted(n for n in os.listdir(CSRC) if n.endswith((".hip", ".hpp", ".cpp", ".h")))
    h = hashlib.sha256()
    for name in names:
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    with open(os.path.join(os.path.dirname(CSRC), "build.py"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()


def step_counter_traffic(wl, tag: str = "") -> tuple:
    """(bytes per step, file) from profiles/step_<workload><tag>_traffic.txt,
    the FETCH_SIZE + WRITE_SIZE counters summed over every kernel of one step,
    when taken on the current library sources; (None, reason) else."""
    path = os.path.join(PROFILES, "step_%s%s_traffic.txt" % (wl.name, tag))
    if not os.path.exists(path):
        return None, "no step counter summary"
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_sources_digest(None):
        return None, "library sources changed since the counters were taken"
    try:
        return int(fields["step_traffic_bytes"]), os.path.relpath(path, ROOT)
    except (KeyError, ValueError):
        return None, "malformed step counter summary"


def host_cpu() -> dict:
    """The host CPU model and the cores this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "nproc": usable, "cpu_count": os.cpu_count()}


def counter_traffic(kernel: str, wl) -> tuple:
    """(bytes per launch, file) from profiles/<kernel>_<workload>_traffic.txt
    when that summary was taken on the current sources; (None, reason) else."""
    path = os.path.join(PROFILES, "%s_%s_traffic.txt" % (kernel, wl.name))
    if not os.path.exists(path):
        return None, "no counter summary"
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != kernel_sources_digest(kernel):
        return None, "kernel sources changed since the counters were taken"
    try:
        return int(fields["traffic_bytes_per_launch"]), os.path.relpath(path, ROOT)
    except (KeyError, ValueError):
        return None, "malformed counter summary"


# ----------------------------------------------------------------------------
# CPU baseline: the fp64 oracle on a bounded sample
# ----------------------------------------------------------------------------

CPU_TARGET_S = 10.0          # repeat the sample until this much oracle time
CPU_MAX_REPEATS = 50
CPU_MEM_BYTES = 8 << 30      # host memory the fp64 sample may take


def _np64(t):
    return t.detach().to("cpu").double().numpy()


def cpu_baseline_planes(wl, inp, oracle, gy=None, merge=None) -> dict:
    """Whole (n, c) planes through the oracle's four-direction forward (or,
    given dL/dy, its backward), each plane run as its own image; repeated
    until CPU_TARGET_S, extrapolated to the workload's n * c planes.  With
    merge weights every sampled plane takes those of channel 0 (the cost does
    not depend on their values)."""
    planes = wl.n * wl.c
    per_plane = (6 + (0 if wl.shared_w else 12)) * wl.h * wl.w * 8 * (2 if gy is not None else 1)
    sample = max(1, min(planes, CPU_MEM_BYTES // per_plane))
    if sample >= 16:
        sample -= sample % 16
    step = max(1, planes // sample)
    idx = [((p * step) // wl.c, (p * step) % wl.c) for p in range(sample)]
    nn = torch.tensor([n for n, _ in idx], device=inp["x"].device)
    cc = torch.tensor([c for _, c in idx], device=inp["x"].device)
    xs = _np64(inp["x"][nn, cc][:, None])
    zs, ls = [], []
    for d in range(4):
        zs.append(_np64(inp["logits"][d][nn, torch.zeros_like(cc) if wl.shared_w else cc][:, None]))
        ls.append(_np64(inp["lam"][d][nn, cc][:, None]))
    gs = _np64(gy[nn, cc][:, None]) if gy is not None else None
    ms = _np64(merge[:, :1]) if merge is not None else None
    reps, spent = 0, 0.0
    while reps < CPU_MAX_REPEATS and (reps == 0 or spent < CPU_TARGET_S):
        t = time.perf_counter()
        if gs is None:
            oracle.forward4(xs, zs, ls, chunk=wl.chunk, merge=ms)
        else:
            oracle.backward4(xs, zs, ls, gs, chunk=wl.chunk, merge=ms)
        spent += time.perf_counter() - t
        reps += 1
    per_call = spent / reps
    what = "forward" if gs is None else "backward"
    threads = min(oracle.max_threads(), sample)  # planes run in parallel (each its own image)
    return {"value": round(per_call * 1e3 * planes / sample, 3), "unit": "ms per %s (extrapolated)" % what,
            "cores": threads, "kind": "oracle", **host_cpu(),
            "sample": "%d of %d planes (%dx%d, every %d-th), each as its own image, all 4 directions, fp64 %s; "
                      "%d runs, %.1f s of oracle time" % (sample, planes, wl.h, wl.w, step, what, reps, spent)}


def cpu_baseline_proxy(wl, inp, oracle, merge=None) -> dict:
    """The whole proxy pipeline once: the down projection over bands of rows,
    the four-direction forward on all proxy planes, the up projection over
    bands of rows (band conversions to fp64 are outside the timed parts)."""
    import numpy as np
    band = 128
    n, c, h, w, cp = wl.n, wl.c, wl.h, wl.w, wl.c_proxy
    wd = _np64(inp["w_down"])
    wu = _np64(inp["w_up"])
    xp = np.empty((n, cp, h, w))
    t_down = t_scan = t_up = 0.0
    for r0 in range(0, h, band):
        xb = np.ascontiguousarray(_np64(inp["x"][:, :, r0:r0 + band]))
        t = time.perf_counter()
        xp[:, :, r0:r0 + band] = oracle.project(xb, wd)
        t_down += time.perf_counter() - t
        del xb
    zs = [_np64(z) for z in inp["logits"]]
    ls = [_np64(l) for l in inp["lam"]]
    t = time.perf_counter()
    yp = oracle.forward4(xp, zs, ls, chunk=wl.chunk, merge=None if merge is None else _np64(merge))
    t_scan = time.perf_counter() - t
    del xp, zs, ls
    for r0 in range(0, h, band):
        yb = np.ascontiguousarray(yp[:, :, r0:r0 + band])
        t = time.perf_counter()
        oracle.project(yb, wu)
        t_up += time.perf_counter() - t
    total = t_down + t_scan + t_up
    return {"value": round(total * 1e3, 3), "unit": "ms per forward", "cores": oracle.max_threads(),
            "kind": "oracle", **host_cpu(),
            "sample": "the whole workload once, fp64: projection down %.2f s and up %.2f s over %d-row bands "
                      "(all threads), four-direction scan of the %d proxy planes %.2f s (%d threads busy)"
                      % (t_down, t_up, band, cp, t_scan, min(oracle.max_threads(), n * cp))}


def cpu_baseline(wl, inp, merge=None) -> dict:
    import oracle
    if wl.c_proxy:
        return cpu_baseline_proxy(wl, inp, oracle, merge)
    return cpu_baseline_planes(wl, inp, oracle, merge=merge)


def copy_rate(mib: int, reps: int = 10) -> tuple:
    """ms per launch and read + write GB/s of a plain device-to-device copy
    of mib MiB."""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    stream = torch.cuda.current_stream()
    b.copy_(a)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(reps):
        b.copy_(a)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    del a, b
    return ms, 2 * n * 4 / (ms * 1e-3) / 1e9


def copy_check(mib: int) -> None:
    """A plain device-to-device copy of known size: reads and writes mib MiB
    per launch.  Used to calibrate the FETCH_SIZE / WRITE_SIZE counters."""
    ms, gbps = copy_rate(mib)
    print(json.dumps({"copy_MiB": mib, "ms": round(ms, 4), "GBps_read_plus_write": round(gbps, 1)}))


def per_step_ms(step, n: int) -> list:
    """Durations (ms) of n single steps, each between its own pair of events
    on the current stream."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in ev)


def cpu_baseline_proxy_backward(wl, inp, gy, oracle, merge=None) -> dict:
    """The oracle's compressive-proxy backward on the workload's top-left
    crop of 1/16 of its pixels (every channel; the cost of each stage is
    linear in the pixel count), repeated until CPU_TARGET_S, scaled to the
    whole plane."""
    hs, ws_ = max(1, wl.h // 4), max(1, wl.w // 4)
    x = _np64(inp["x"][:, :, :hs, :ws_])
    g = _np64(gy[:, :, :hs, :ws_])
    zs = [_np64(z[..., :hs, :ws_] if d < 2 else z[..., :ws_, :hs]) for d, z in enumerate(inp["logits"])]
    ls = [_np64(l[..., :hs, :ws_] if d < 2 else l[..., :ws_, :hs]) for d, l in enumerate(inp["lam"])]
    wd, wu = _np64(inp["w_down"]), _np64(inp["w_up"])
    m = None if merge is None else _np64(merge)
    reps, spent = 0, 0.0
    while reps < CPU_MAX_REPEATS and (reps == 0 or spent < CPU_TARGET_S):
        t = time.perf_counter()
        oracle.proxy_backward4(x, wd, wu, zs, ls, g, chunk=wl.chunk, merge=m)
        spent += time.perf_counter() - t
        reps += 1
    scale = (wl.h * wl.w) / (hs * ws_)
    return {"value": round(spent / reps * 1e3 * scale, 3), "unit": "ms per proxy backward (extrapolated)",
            "cores": oracle.max_threads(), "kind": "oracle", **host_cpu(),
            "sample": "the %dx%d top-left crop (all %d channels, %d proxy channels), fp64 chain-rule backward "
                      "(projections, four-direction forward and backward in proxy space, weight gradients), "
                      "scaled by the pixel ratio %.0f; %d runs, %.1f s of oracle time"
                      % (hs, ws_, wl.c, wl.c_proxy, scale, reps, spent)}


def bench_proxy_backward(args, wl):
    """The backward leg of the compressive-proxy workload:
    gspn_proxy_backward4 for a seeded dL/dy ~ N(0, 1).  The dominant kernel
    is the stage that takes longest (the weight-gradient passes, two
    launches, at full size).  With --pass train a step is a training step:
    gspn_proxy_forward4 keeping its proxy-space state, then
    gspn_proxy_backward4 from it (no recompute)."""
    train = args.pass_ == "train"
    torch.cuda.init()
    G.lib()
    print("bench: proxy %s, workload %s, generating inputs" % ("train" if train else "backward", wl.name),
          file=sys.stderr, flush=True)
    lay = args.layout
    inp = make_inputs(wl, "cuda")
    tin = array_layout(inp) if lay == "array" else inp
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed + 1000)
    gy = torch.randn(inp["x"].shape, generator=g, device="cuda", dtype=torch.float32).to(wl.torch_dtype)
    ws = G.proxy_backward4_workspace(inp["x"], wl.c_proxy, wl.cw, lay)
    merge = merge_weights(wl, args.merge)
    fws = G.proxy_forward4_workspace(inp["x"], wl.c_proxy, wl.cw, lay) if train else None
    kept = G.proxy_states_buffer(inp["x"], wl.c_proxy) if train else None
    y = torch.empty_like(inp["x"]) if train else None
    ftimes = {}

    def step(times=None):
        args_ = (tin["x"], tin["w_down"], tin["w_up"], tin["logits"], tin["lam"])
        if train:
            if times is not None:
                _, ftimes["t"] = G.gspn_proxy_forward4_timed(*args_, chunk_len=wl.chunk, out=y, workspace=fws,
                                                             merge=merge, layout=lay, states=kept)
            else:
                G.gspn_proxy_forward4(*args_, chunk_len=wl.chunk, out=y, workspace=fws, merge=merge, layout=lay,
                                      states=kept)
        return G.gspn_proxy_backward4(*args_, gy, chunk_len=wl.chunk, workspace=ws, times=times, merge=merge,
                                      layout=lay, states=kept)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    print("bench: proxy %s %.3f ms/step" % ("train" if train else "backward", ms), file=sys.stderr, flush=True)
    singles = per_step_ms(step, args.steps)
    reps = max(3, min(args.steps, 10))
    acc = {name: [0.0, 0] for name in G.STAGES}
    facc = {name: [0.0, 0] for name in G.STAGES}
    for _ in range(reps):
        t = G.StageTimes()
        step(times=t)
        for name, v in t.as_dict().items():
            if name in acc:
                acc[name][0] += v["ms"] / reps
                acc[name][1] = v["launches"]
        for name, v in ftimes.get("t", {}).items():
            if name in facc:
                facc[name][0] += v["ms"] / reps
                facc[name][1] = v["launches"]
    stage = max(("weight_grad", "project_down", "project_up"), key=lambda k: acc[k][0])
    launches = acc[stage][1]
    kernel_ms = acc[stage][0] / launches
    if stage == "weight_grad":
        kernel, bpl = "wgrad_mfma", wgrad_pass_bytes(wl)
        slots = min(2048, wl.n * wl.h * wl.w // 128)
        design = bpl + slots * wl.c * wl.c_proxy * 4      # plus each pass's fp32 partial sums
    else:
        kernel = PROJECTION_KERNELS[stage]
        bpl = design = projection_bytes(wl, stage == "project_down")
    achieved = bpl / (kernel_ms * 1e-3) / 1e9
    alg = proxy_backward_bytes(wl) + (algorithmic_bytes(wl) if train else 0)
    eff = alg / (ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle's proxy backward on a sample", file=sys.stderr, flush=True)
        import oracle
        cpu = cpu_baseline_proxy_backward(wl, inp, gy, oracle, merge)
    traffic, traffic_src = counter_traffic(kernel, wl) if lay == "scan" else (None, "scan layout only")
    tag = ("_train" if train else "_backward") + ("" if lay == "scan" else "_array")
    step_traffic, step_src = step_counter_traffic(wl, tag)
    grads = "dx, dw_down, dw_up, dlambda, dlogits%s" % (", dmerge" if args.merge else "")
    if train:
        stages = {"forward_" + k: round(v[0], 4) for k, v in facc.items() if v[1]}
        stages.update({"backward_" + k: round(v[0], 4) for k, v in acc.items() if v[1]})
    else:
        stages = {k: round(v[0], 4) for k, v in acc.items() if v[1]}
    rec = {
        "metric": ("ms per compressive-proxy GSPN training step (forward keeping its proxy-space state, then "
                   "backward: %s); achieved HBM GB/s" % grads) if train else
                  ("ms per compressive-proxy GSPN backward (%s); achieved HBM GB/s" % grads),
        "value": round(ms, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded)",
        "config": {"workload": wl.name, "pass": "train" if train else "backward", "n": wl.n, "c": wl.c,
                   "h": wl.h, "w": wl.w, "storage": wl.dtype, "shared_w": wl.shared_w, "chunk_len": wl.chunk,
                   "c_proxy": wl.c_proxy, "merge": "learnable" if args.merge else "sum", "layout": lay},
        "ms_median": round(singles[len(singles) // 2], 4), "ms_min": round(singles[0], 4),
        "effective_GBps": round(eff, 1), "effective_frac": round(eff / HBM_PEAK_GBPS, 4), "algorithmic_bytes": alg,
        "stages_ms": stages,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": kernel,
                     "kernel_ms": round(kernel_ms, 4), "launches_per_step": launches, "bytes_per_launch": bpl,
                     "traffic_source": traffic_src, "design_bytes_per_launch": design,
                     "design_achieved": round(design / (kernel_ms * 1e-3) / 1e9, 1),
                     "step_traffic": step_traffic, "step_traffic_source": step_src},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))


def bench_backward(args, wl):
    """The backward leg: gspn_backward4 over the same inputs and a seeded
    dL/dy ~ N(0, 1); the dominant kernel is the adjoint launch.  With
    --pass train a step is a training step instead: gspn_forward4 keeping
    its fp32 states, then gspn_backward4 from those states (no recompute)."""
    train = args.pass_ == "train"
    if wl.c_proxy:
        bench_proxy_backward(args, wl)
        return
    if train and wl.h <= 64 and wl.w <= 64:
        print("bench.py: the forward keeps its states only for planes larger than 64 x 64", file=sys.stderr)
        sys.exit(2)
    torch.cuda.init()
    G.lib()
    print("bench: backward, workload %s, generating inputs" % wl.name, file=sys.stderr, flush=True)
    lay = args.layout
    inp = make_inputs(wl, "cuda")            # scan frame (also what the CPU oracle reads)
    tin = array_layout(inp) if lay == "array" else inp
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed + 1000)
    gy = torch.randn(inp["x"].shape, generator=g, device="cuda", dtype=torch.float32).to(wl.torch_dtype)
    outs = (torch.empty_like(inp["x"]), [torch.empty_like(z) for z in tin["logits"]],
            [torch.empty_like(l) for l in tin["lam"]])
    ws = G.backward4_workspace(inp["x"], wl.cw, with_states=train, layout=lay)
    merge = merge_weights(wl, args.merge)
    dmerge = torch.empty((4, wl.c_scan), dtype=torch.float32, device="cuda") if args.merge else None
    fws = G.forward4_workspace(inp["x"], wl.cw, lay) if train else None
    states = G.states_buffer(inp["x"]) if train else None
    y = torch.empty_like(inp["x"]) if train else None

    def step(times=None, ftimes=None):
        if train:
            if ftimes is None:
                G.gspn_forward4(tin["x"], tin["logits"], tin["lam"], chunk_len=wl.chunk, out=y, workspace=fws,
                                merge=merge, states=states, layout=lay)
            else:
                _, ft = G.gspn_forward4_timed(tin["x"], tin["logits"], tin["lam"], chunk_len=wl.chunk, out=y,
                                              workspace=fws, merge=merge, states=states, layout=lay)
                ftimes.update(ft)
        return G.gspn_backward4(tin["x"], tin["logits"], tin["lam"], gy, chunk_len=wl.chunk, workspace=ws,
                                out=outs, times=times, merge=merge, dmerge=dmerge, states=states, layout=lay)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    print("bench: %s %.3f ms/step" % (args.pass_, ms), file=sys.stderr, flush=True)
    singles = per_step_ms(step, args.steps)

    reps = max(3, min(args.steps, 10))
    acc = {name: 0.0 for name in G.STAGES}
    facc = {name: 0.0 for name in G.STAGES}
    recompute = None
    adj_plan, adj_launches = None, 1
    for _ in range(reps):
        t = G.StageTimes()
        ft = {}
        step(times=t, ftimes=ft if train else None)
        for name, v in t.as_dict().items():
            if name == "scan_kernel":
                recompute = v
            elif name == "adjoint_plan":
                adj_plan = v
            else:
                acc[name] += v["ms"] / reps
                if name == "adjoint":
                    adj_launches = max(1, v["launches"])
        for name, v in ft.items():
            if name not in ("scan_kernel", "adjoint_plan"):
                facc[name] += v["ms"] / reps
    kernel_ms = acc["adjoint"] / adj_launches
    # planes of at most 64 x 64 recompute with the plane-resident forward
    # and run the plane-resident adjoint; very few long lines run the banded
    # adjoint, one launch per band
    adj_kernel = "adjplane_kernel" if recompute == "plane4_kernel" else "adj4_kernel"
    if adj_plan is not None and adj_plan["kernel"] == "adj4band_kernel":
        adj_kernel = "adj4band_kernel"
    design = adjplane_launch_bytes(wl) if adj_kernel == "adjplane_kernel" else adjoint_launch_bytes(wl)
    design //= adj_launches
    # the adjoint launches process every unit of the backward: its compulsory bytes
    bpl = backward_algorithmic_bytes(wl) // adj_launches
    achieved = bpl / (kernel_ms * 1e-3) / 1e9
    alg = backward_algorithmic_bytes(wl) + (algorithmic_bytes(wl) if train else 0)
    eff = alg / (ms * 1e-3) / 1e9
    stages = {k: round(v, 4) for k, v in acc.items() if v > 0}
    if train:
        stages = dict([("forward_" + k, round(v, 4)) for k, v in facc.items() if v > 0] +
                      [("backward_" + k, v) for k, v in stages.items()])
    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle's backward on a sample", file=sys.stderr, flush=True)
        import oracle
        cpu = cpu_baseline_planes(wl, inp, oracle, gy=gy, merge=merge)
    traffic, traffic_src = counter_traffic(adj_kernel, wl) if lay == "scan" else (None, "scan layout only")
    tag = ("_train" if train else "_backward") + ("" if lay == "scan" else "_array")
    step_traffic, step_src = step_counter_traffic(wl, tag)
    rec = {
        "metric": ("ms per 4-direction GSPN training step (forward keeping fp32 states, then backward: dx, "
                   "dlambda, dlogits%s); achieved HBM GB/s" if train else
                   "ms per 4-direction GSPN backward (dx, dlambda, dlogits%s); achieved HBM GB/s")
                  % (", dmerge" if args.merge else ""),
        "value": round(ms, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded)",
        "config": {"workload": wl.name, "pass": args.pass_, "n": wl.n, "c": wl.c, "h": wl.h, "w": wl.w,
                   "storage": wl.dtype, "shared_w": wl.shared_w, "chunk_len": wl.chunk,
                   "merge": "learnable" if args.merge else "sum", "layout": lay},
        "ms_median": round(singles[len(singles) // 2], 4), "ms_min": round(singles[0], 4),
        "effective_GBps": round(eff, 1), "effective_frac": round(eff / HBM_PEAK_GBPS, 4), "algorithmic_bytes": alg,
        "stages_ms": stages,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": adj_kernel,
                     "kernel_ms": round(kernel_ms, 4), "launches_per_step": adj_launches, "bytes_per_launch": bpl,
                     "traffic_source": traffic_src, "design_bytes_per_launch": design,
                     "design_achieved": round(design / (kernel_ms * 1e-3) / 1e9, 1),
                     "step_traffic": step_traffic, "step_traffic_source": step_src},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="profile", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="pass_", default="forward", choices=("forward", "backward", "train"),
                    help="time the forward (default), the backward (gradients for a seeded dL/dy), or a "
                         "training step (forward keeping its states, then the backward from them)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays (forward only)")
    ap.add_argument("--merge", action="store_true",
                    help="merge the directions with seeded learnable weights per direction and channel")
    ap.add_argument("--layout", default="scan", choices=("scan", "array"),
                    help="per-direction logits / lambdas in their scan frames (default) or all in the array "
                         "frame [.., H, W] (the library then copies the horizontal ones inside the step)")
    ap.add_argument("--copy-check", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the four-direction scan has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    if args.copy_check:
        copy_check(args.copy_check)
        return
    wl = WORKLOADS[args.workload]
    if args.pass_ in ("backward", "train"):
        bench_backward(args, wl)
        return
    torch.cuda.init()
    G.lib()
    print("bench: workload %s, generating inputs" % wl.name, file=sys.stderr, flush=True)
    lay = args.layout
    inp = make_inputs(wl, "cuda")            # scan frame (also what the CPU oracle reads)
    tin = array_layout(inp) if lay == "array" else inp
    out = torch.empty_like(inp["x"])
    ws = (G.proxy_forward4_workspace(inp["x"], wl.c_proxy, wl.cw, lay) if wl.c_proxy
          else G.forward4_workspace(inp["x"], wl.cw, lay))
    merge = merge_weights(wl, args.merge)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        run_step(wl, tin, out, ws, merge=merge, layout=lay)
    torch.cuda.synchronize()
    step = lambda: run_step(wl, tin, out, ws, merge=merge, layout=lay)
    if args.graph:
        # the library allocates nothing and launches only kernels on the
        # current stream, so one step captures whole; its replays are timed
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run_step(wl, tin, out, ws, merge=merge, layout=lay)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_step(wl, tin, out, ws, merge=merge, layout=lay)
        torch.cuda.synchronize()
        step = graph.replay
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / args.steps
    print("bench: %.3f ms/step (wall %.3f ms/step)" % (ms, wall * 1e3 / args.steps),
          file=sys.stderr, flush=True)

    singles = per_step_ms(step, args.steps)
    st, kernel = stage_times(wl, tin, out, ws, reps=max(3, min(args.steps, 10)), merge=merge, layout=lay)
    scan = st["scan"]
    launches = scan["launches"]
    kernel_ms = scan["ms"] / launches
    bpl = launch_algorithmic_bytes(wl, launches)
    design = scan_launch_bytes(wl, kernel, launches)
    if kernel == "seq4_kernel" and st["tail"]["launches"]:
        # the launch covers all but the tail's planes
        planes = wl.n * wl.c_scan
        run = seq4_launch_planes(wl, torch.cuda.get_device_properties(0).multi_processor_count, True)
        bpl = bpl * run // planes
        design = design * run // planes
    scan_roofline = None
    if wl.c_proxy:
        # the dominant kernel is the stage that takes longest: in the proxy
        # pipeline a projection (one launch each); the scan's figures are
        # kept beside it
        scan_achieved = bpl / (kernel_ms * 1e-3) / 1e9
        scan_roofline = {"kernel": kernel, "kernel_ms": round(kernel_ms, 4), "launches_per_step": launches,
                         "bytes_per_launch": bpl, "achieved": round(scan_achieved, 1),
                         "frac": round(scan_achieved / HBM_PEAK_GBPS, 4), "design_bytes_per_launch": design}
        stage = max(("project_down", "project_up", "scan"), key=lambda k: st[k]["ms"])
        if stage != "scan":
            kernel = PROJECTION_KERNELS[stage]
            launches = st[stage]["launches"]
            kernel_ms = st[stage]["ms"] / launches
            bpl = design = projection_bytes(wl, stage == "project_down")
    achieved = bpl / (kernel_ms * 1e-3) / 1e9
    tag = "" if lay == "scan" else "_array"
    traffic, traffic_src = counter_traffic(kernel, wl) if lay == "scan" else (None, "scan layout only")
    step_traffic, step_src = step_counter_traffic(wl, tag)
    alg = algorithmic_bytes(wl)
    eff = alg / (ms * 1e-3) / 1e9
    print("bench: %s %.4f ms per launch (%d per step), %.1f GB/s algorithmic"
          % (kernel, kernel_ms, launches, achieved), file=sys.stderr, flush=True)

    # a 4 GiB device copy (8 GiB moved) on the same GPU, for scale
    _, copy_gbps = copy_rate(4096, reps=5)

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, inp, merge)

    rec = {
        "metric": METRIC if not args.merge else METRIC.replace("forward", "forward (learnable merge)"),
        "value": round(ms, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded)",
        "config": {"workload": wl.name, "n": wl.n, "c": wl.c, "h": wl.h, "w": wl.w,
                   "storage": wl.dtype, "shared_w": wl.shared_w, "chunk_len": wl.chunk,
                   "c_proxy": wl.c_proxy, "merge": "learnable" if args.merge else "sum",
                   "launch": "hip graph replay" if args.graph else "eager", "layout": lay},
        "ms_median": round(singles[len(singles) // 2], 4),
        "ms_min": round(singles[0], 4),
        "effective_GBps": round(eff, 1),
        "effective_frac": round(eff / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes": alg,
        "copy_GBps": round(copy_gbps, 1),
        "effective_frac_of_copy": round(eff / copy_gbps, 4),
        "achieved_frac_of_copy": round(achieved / copy_gbps, 4),
        "stages_ms": {k: round(v["ms"], 4) for k, v in st.items() if v["launches"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": kernel, "kernel_ms": round(kernel_ms, 4), "launches_per_step": launches,
                     "bytes_per_launch": bpl, "traffic_source": traffic_src,
                     "design_bytes_per_launch": design,
                     "design_achieved": round(design / (kernel_ms * 1e-3) / 1e9, 1),
                     "step_traffic": step_traffic, "step_traffic_source": step_src},
        "cpu_baseline": cpu,
    }
    if scan_roofline is not None:
        rec["scan_roofline"] = scan_roofline
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
