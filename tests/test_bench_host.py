"""CPU tests of bench.py's host logic: the byte models that roofline.achieved
and the effective bandwidth divide by, their agreement with the library's own
workspace layout, the gate that reports counter traffic only for the sources
it was measured on, and the refusal of more than one GPU.

The expected byte counts are written out from the definitions (every distinct
input read once and y written once; for a scan launch, every tensor it reads
or writes moved once), not taken from bench.py."""
import os
import subprocess
import sys

import pytest

import bench
from linear_spatial_propagation_gspn_amd import gspn as G
from linear_spatial_propagation_gspn_amd.workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# Compulsory bytes of one forward step, per workload:
#   per-channel logits, fp32 (profile, tstage): x + 4 lambdas + 4 x 3 logits + y = 18 U;
#   channel-shared logits (wide): x + 4 lambdas + y in bf16, one logit triple per position;
#   proxy: x and y at C = 320, the proxy-space lambdas and logits, both projection matrices.
@pytest.mark.parametrize("name,expected", [
    ("profile", 18 * 16 * 8 * 1024 * 1024 * 4),                                  # 9,663,676,416
    ("tstage", 18 * 64 * 96 * 56 * 56 * 4),                                      # 1,387,266,048
    ("tstage_chunk8", 18 * 64 * 96 * 56 * 56 * 4),
    ("wide", 6 * 1152 * 1024 * 1024 * 2 + 4 * 3 * 1024 * 1024 * 2),            # 14,520,680,448
    ("proxy", 2 * 320 * 2048 * 2048 * 2 + 4 * 8 * 2048 * 2048 * 2 + 4 * 3 * 2048 * 2048 * 2
     + 2 * 320 * 8 * 2),                                                          # 5,737,818,112
])
def test_forward_algorithmic_bytes(name, expected):
    assert bench.algorithmic_bytes(WORKLOADS[name]) == expected


def test_scan_launch_bytes():
    u = 16 * 8 * 1024 * 1024 * 4
    # long-line launch: x and x transposed, 4 x 3 logit planes, 4 lambdas, 4 maps written
    assert bench.scan_launch_bytes(WORKLOADS["profile"], "scan4lp_kernel") == 22 * u
    # plane kernel: compulsory bytes only
    t = 64 * 96 * 56 * 56 * 4
    assert bench.scan_launch_bytes(WORKLOADS["tstage"], "plane4_kernel") == 18 * t
    # channel-shared bf16 weights reach the scan as packed half pairs, 4 bytes a position
    uw = 1152 * 1024 * 1024 * 2
    assert bench.scan_launch_bytes(WORKLOADS["wide"], "scan4lp_kernel") == 10 * uw + 4 * 1024 * 1024 * 4
    # plane-sequential kernel on the wide workload: x four times, lambdas and
    # half-pair weights once, z 4U, y 3U
    assert bench.scan_launch_bytes(WORKLOADS["wide"], "seq4_kernel") == 15 * uw + 4 * 1024 * 1024 * 4
    # 1152 planes on 256 CUs: the last 128 go to the concurrent path
    assert bench.seq4_launch_planes(WORKLOADS["wide"], 256, True) == 1024
    assert bench.seq4_launch_planes(WORKLOADS["wide"], 256, False) == 1152
    # banded scan of the 8 proxy planes: the same launch's bytes over its 16 bands
    up = 8 * 2048 * 2048 * 2
    assert bench.scan_launch_bytes(WORKLOADS["proxy"], "scan4band_kernel", 16) == \
        (10 * up + 4 * 2048 * 2048 * 4) // 16


@pytest.mark.parametrize("name", ["wide", "proxy", "profile"])
def test_weight_bytes_follow_the_library_workspace(name):
    """The weights the scans read are what gspn_forward4 keeps in its
    workspace: with channel-shared logits over several channels the workspace
    grows by exactly the four directions' normalised weights."""
    wl = WORKLOADS[name]
    lib = G.lib()
    dt = 0 if wl.dtype == "f32" else 1
    c = wl.c_scan
    shared = lib.gspn_forward4_workspace_bytes(wl.n, c, wl.h, wl.w, 1, dt, 0)
    per_channel = lib.gspn_forward4_workspace_bytes(wl.n, c, wl.h, wl.w, c, dt, 0)
    if bench.prenormalised(wl):
        assert shared - per_channel == 4 * bench.weight_bytes_per_direction(wl)
    else:
        assert bench.weight_bytes_per_direction(wl) == wl.n * wl.cw * 3 * wl.h * wl.w * bench.esize(wl)


def _summary(path, sha, traffic=123456):
    with open(path, "w") as f:
        f.write("# test summary\nkernel: k\ntraffic_bytes_per_launch: %d\nsource_sha256: %s\n" % (traffic, sha))


def test_counter_traffic_only_for_the_measured_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    wl = WORKLOADS["profile"]
    assert bench.counter_traffic("scan4lp_kernel", wl) == (None, "no counter summary")
    path = tmp_path / "scan4lp_kernel_profile_traffic.txt"
    _summary(path, bench.kernel_sources_digest("scan4lp_kernel"))
    value, src = bench.counter_traffic("scan4lp_kernel", wl)
    assert value == 123456 and src.endswith("scan4lp_kernel_profile_traffic.txt")
    _summary(path, "0" * 64)
    assert bench.counter_traffic("scan4lp_kernel", wl) == \
        (None, "kernel sources changed since the counters were taken")


def test_kernel_digests_cover_their_sources():
    # every measured kernel hashes its own sources; the banded kernel's include
    # the long-line kernel's, whose device code it reuses
    for k in bench.KERNEL_SOURCES:
        assert len(bench.kernel_sources_digest(k)) == 64
    assert bench.kernel_sources_digest("scan4band_kernel") != bench.kernel_sources_digest("scan4lp_kernel")
    assert set(bench.KERNEL_SOURCES["scan4lp_kernel"]) <= set(bench.KERNEL_SOURCES["scan4band_kernel"])


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_scan_algorithmic_bytes_are_the_compulsory_bytes():
    """roofline.frac is taken on the four-direction scan's compulsory bytes
    (every distinct input read once as stored, y written once): 18U for fp32
    per-channel logits (9,663,676,416 bytes on 1024^2, B=16, C=8) and
    6U + 12 N H W 2 bytes for bf16 channel-shared logits (14,520,680,448 on
    1024^2, B=1, C=1152), divided over the launches that share the scan."""
    assert bench.scan_algorithmic_bytes(WORKLOADS["profile"]) == 9663676416
    assert bench.scan_algorithmic_bytes(WORKLOADS["profile"]) == bench.algorithmic_bytes(WORKLOADS["profile"])
    assert bench.scan_algorithmic_bytes(WORKLOADS["wide"]) == 14520680448
    assert bench.scan_algorithmic_bytes(WORKLOADS["tstage"]) == 1387266048
    up = 8 * 2048 * 2048 * 2  # one proxy-space map
    assert bench.scan_algorithmic_bytes(WORKLOADS["proxy"]) == 6 * up + 4 * 3 * 2048 * 2048 * 2
    assert bench.launch_algorithmic_bytes(WORKLOADS["proxy"], 16) == (6 * up + 4 * 3 * 2048 * 2048 * 2) // 16
    assert bench.launch_algorithmic_bytes(WORKLOADS["profile"], 1) == 9663676416


def test_projection_bytes():
    # proxy: 320 -> 8 channels over 2048^2 bf16 pixels, and the weights
    px = 2048 * 2048
    assert bench.projection_bytes(WORKLOADS["proxy"], True) == (320 + 8) * px * 2 + 320 * 8 * 2
    assert bench.projection_bytes(WORKLOADS["proxy"], False) == bench.projection_bytes(WORKLOADS["proxy"], True)
    assert set(bench.PROJECTION_KERNELS.values()) <= set(bench.KERNEL_SOURCES)


def test_host_cpu_fields():
    info = bench.host_cpu()
    assert set(info) == {"cpu_model", "nproc", "cpu_count"}
    assert info["nproc"] >= 1
