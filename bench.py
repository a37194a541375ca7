"""Benchmark of the four-direction GSPN line-scan forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload profile]

A step is one gspn_forward4 call (normalise the logits, scan T->B, B->T,
L->R, R->L, merge by summation) over one batch of seeded synthetic inputs
already resident in HBM; for the proxy workload a step is the compressive
proxy pipeline (1x1 projection down, forward4 in proxy space, 1x1 projection
up).  Prints one JSON line.

Measurements:
  - ms per step: HIP events on the stream the library launches on, bracketing
    the K timed steps (synchronised on both sides).
  - roofline: the dominant kernel (the line-scan kernel) timed per launch with
    HIP events in its own loop over the same inputs and launch configuration;
    achieved = its algorithmic bytes per launch / its average duration.
  - effective bandwidth of the whole step = algorithmic bytes of the forward
    (every distinct input read once, y written once) / ms per step.
  - cpu_baseline: the fp64 oracle on a bounded sample of the same workload,
    on the host's cores (rank 0, N = 1 only).
"""
from __future__ import annotations

import argparse
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


def esize(wl) -> int:
    return 4 if wl.dtype == "f32" else 2


def algorithmic_bytes(wl) -> int:
    """Every distinct input read once and y written once."""
    es = esize(wl)
    hw = wl.h * wl.w
    if wl.c_proxy:
        x = wl.n * wl.c * hw * es
        y = x
        lam = 4 * wl.n * wl.c_proxy * hw * es
        z = 4 * wl.n * wl.cw * 3 * hw * es
        wts = 2 * wl.c * wl.c_proxy * es
        return x + y + lam + z + wts
    u = wl.n * wl.c * hw * es
    z = 4 * wl.n * wl.cw * 3 * hw * es
    return u + 4 * u + z + u


def scan_launch_bytes(wl, accumulate: bool) -> int:
    """Compulsory bytes of one direction's scan launch: x, its logits and
    lambda read once, the output written once (and read once when the launch
    accumulates into it)."""
    es = esize(wl)
    c = wl.c_scan
    u = wl.n * c * wl.h * wl.w * es
    z = wl.n * wl.cw * 3 * wl.h * wl.w * es
    return u + z + u + u + (u if accumulate else 0)


def scan4_launch_bytes(wl) -> int:
    """Compulsory bytes of one four-direction launch: x once, the four
    directions' logits and lambda once, four output maps written once."""
    es = esize(wl)
    u = wl.n * wl.c_scan * wl.h * wl.w * es
    z = wl.n * wl.cw * 3 * wl.h * wl.w * es
    return u + 4 * z + 4 * u + 4 * u


# Mirror of the library's rule (api.cpp): with a workspace, gspn_forward4 runs
# the four directions in one launch when one direction has fewer than 512
# (plane, chunk) lines and no line exceeds 2048 positions.
def uses_fused_path(wl) -> bool:
    most = 0
    for S in (wl.h, wl.w):
        k = S if wl.chunk in (0,) or wl.chunk >= S else wl.chunk
        most = max(most, wl.n * wl.c_scan * ((S + k - 1) // k))
    return most < 512 and max(wl.h, wl.w) <= 2048


def run_step(wl, inp, out, ws):
    if wl.c_proxy:
        return G.gspn_proxy_forward4(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"],
                                     chunk_len=wl.chunk, out=out, workspace=ws)
    return G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], chunk_len=wl.chunk, out=out,
                           workspace=ws)


def _time(fn, reps: int) -> float:
    """Average ms of fn() over reps launches, HIP events on the current stream."""
    stream = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / reps


def time_dominant_kernel(wl, inp, reps: int) -> dict:
    """Per-launch duration of the scan kernel in the configuration the step uses."""
    x = G.gspn_proxy_project(inp["x"], inp["w_down"]) if wl.c_proxy else inp["x"]
    if uses_fused_path(wl):
        outs = [torch.empty_like(x) for _ in range(4)]
        ms = _time(lambda: G.gspn_scan4_fwd(x, inp["logits"], inp["lam"], wl.chunk, outs), reps)
        return {"kernel": "scan4_kernel", "kernel_ms": ms, "bytes_per_launch": scan4_launch_bytes(wl)}
    out = torch.empty_like(x)
    per_dir, total_bytes = [], 0
    for d in range(4):
        acc = d > 0
        ms = _time(lambda: G.gspn_scan_fwd(d, x, inp["logits"][d], inp["lam"][d], wl.chunk, out=out,
                                           accumulate=acc), reps)
        per_dir.append(ms)
        total_bytes += scan_launch_bytes(wl, acc)
    return {"kernel": "scan_kernel", "kernel_ms": sum(per_dir) / 4, "bytes_per_launch": total_bytes // 4,
            "per_direction_ms": [round(m, 4) for m in per_dir]}


def cpu_baseline(wl, inp):
    """The fp64 oracle on a bounded sample of the workload (whole planes),
    scaled to ms per full forward."""
    import oracle
    nthreads = os.cpu_count() or 1
    planes = wl.n * wl.c
    if wl.c_proxy:
        # sample: the proxy-space four-direction scan (all proxy planes) plus
        # the two projections restricted to a pixel band
        return None
    budget_planes = max(1, min(planes, 16 if wl.h * wl.w >= 1 << 20 else 512))
    idx = [(p // wl.c, p % wl.c) for p in range(budget_planes)]
    xs = torch.stack([inp["x"][n, c] for n, c in idx])[:, None].float().cpu()
    zs, ls = [], []
    for d in range(4):
        zs.append(torch.stack([inp["logits"][d][n, 0 if wl.shared_w else c] for n, c in idx])[:, None]
                  .float().cpu())
        ls.append(torch.stack([inp["lam"][d][n, c] for n, c in idx])[:, None].float().cpu())
    t = time.perf_counter()
    oracle.forward4(xs, zs, ls, chunk=wl.chunk)
    dt = time.perf_counter() - t
    ms_full = dt * 1e3 * planes / budget_planes
    return {"value": round(ms_full, 3), "unit": "ms per forward (extrapolated)", "cores": nthreads,
            "kind": "oracle",
            "sample": "%d of %d planes (%dx%d), all 4 directions, fp64, %.2f s measured"
                      % (budget_planes, planes, wl.h, wl.w, dt)}


def copy_check(mib: int) -> None:
    """A plain device-to-device copy of known size: reads and writes mib MiB
    per launch.  Used to calibrate the FETCH_SIZE / WRITE_SIZE counters."""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    ms = _time(lambda: b.copy_(a), 10)
    print(json.dumps({"copy_MiB": mib, "ms": round(ms, 4),
                      "GBps_read_plus_write": round(2 * n * 4 / (ms * 1e-3) / 1e9, 1)}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="profile", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-check", type=int, default=0, metavar="MIB",
                    help="only run a device-to-device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus must be 1)",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_check:
        copy_check(args.copy_check)
        return
    wl = WORKLOADS[args.workload]
    torch.cuda.init()
    G.lib()
    print("bench: workload %s, generating inputs" % wl.name, file=sys.stderr, flush=True)
    inp = make_inputs(wl, "cuda")
    out = torch.empty_like(inp["x"])
    ws = (G.proxy_forward4_workspace(inp["x"], wl.c_proxy, wl.cw) if wl.c_proxy
          else G.forward4_workspace(inp["x"], wl.cw))
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        run_step(wl, inp, out, ws)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        run_step(wl, inp, out, ws)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(stop) / args.steps
    print("bench: %.3f ms/step (wall %.3f ms/step)" % (ms, wall * 1e3 / args.steps),
          file=sys.stderr, flush=True)

    dom = time_dominant_kernel(wl, inp, reps=max(3, min(args.steps, 10)))
    achieved = dom["bytes_per_launch"] / (dom["kernel_ms"] * 1e-3) / 1e9
    alg = algorithmic_bytes(wl)
    eff = alg / (ms * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, inp)

    rec = {
        "metric": METRIC,
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
                   "c_proxy": wl.c_proxy},
        "effective_GBps": round(eff, 1),
        "effective_frac": round(eff / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes": alg,
        "roofline": dict({"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                          "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None},
                         **{k: (round(v, 4) if isinstance(v, float) else v) for k, v in dom.items()}),
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
