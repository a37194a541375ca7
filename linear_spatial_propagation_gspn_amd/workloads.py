"""Seeded synthetic inputs shaped like the GSPN pages' workloads.

This module draws random tensors and nothing else: it holds none of the
propagation's arithmetic, so both the HIP path and the CPU oracle can consume
its output.  Values are drawn in float32 with a seeded ``torch.Generator``
and, for bf16 workloads, rounded once to bfloat16 (round to nearest even);
both sides then read the same stored values.

Draw order (fixed): x; then for each direction T2B, B2T, L2R, R2L: its
logits, then its lambda; then W_down, W_up (proxy workloads only).

Distributions: x ~ N(0, 1); logits ~ N(0, 1); lambda ~ U(0, 1);
W_down ~ N(0, sd 1/sqrt(C)); W_up ~ N(0, sd 1/sqrt(C_proxy)).

Per-direction tensors are laid out in the direction's scan frame:
logits [N][Cw][3][S][L], lambda [N][Cs][S][L] with (S, L) = (H, W) for the
vertical directions and (W, H) for the horizontal ones; Cs is the number of
channels the scan runs on (C, or C_proxy for proxy workloads) and Cw is 1
(channel-shared w) or Cs (per-channel w).

Named workloads (sizes from the GSPN-2 pages' profiling shapes and GSPN-T
stage maps):
  tiny     N=1,  C=2,    16x16,     fp32, per-channel w
  tstage   N=64, C=96,   56x56,     fp32, per-channel w (also chunk_len=8)
  profile  N=16, C=8,    1024x1024, fp32, per-channel w
  wide     N=1,  C=1152, 1024x1024, bf16, channel-shared w
  proxy    N=1,  C=320,  2048x2048, bf16, channel-shared w, C_proxy=8
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

DIRECTIONS = ("T2B", "B2T", "L2R", "R2L")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n: int
    c: int
    h: int
    w: int
    dtype: str = "f32"          # storage type: "f32" or "bf16"
    shared_w: bool = False      # channel-shared w (one logit triple per position)
    chunk: int = 0              # 0 = full-length scan
    seed: int = 0
    c_proxy: int = 0            # >0: compressive proxy workload

    @property
    def c_scan(self) -> int:
        return self.c_proxy if self.c_proxy > 0 else self.c

    @property
    def cw(self) -> int:
        return 1 if self.shared_w else self.c_scan

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def frame(self, d: int) -> tuple[int, int]:
        return (self.w, self.h) if d >= 2 else (self.h, self.w)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 16, 16, "f32", False, 0, 1),
    "tstage": Workload("tstage", 64, 96, 56, 56, "f32", False, 0, 2),
    "tstage_chunk8": Workload("tstage_chunk8", 64, 96, 56, 56, "f32", False, 8, 2),
    "profile": Workload("profile", 16, 8, 1024, 1024, "f32", False, 0, 3),
    "wide": Workload("wide", 1, 1152, 1024, 1024, "bf16", True, 0, 4),
    "proxy": Workload("proxy", 1, 320, 2048, 2048, "bf16", True, 0, 5, c_proxy=8),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def make_inputs(wl: Workload, device="cpu", seed: Optional[int] = None) -> dict:
    """Draw every input of a workload on ``device`` in the fixed order.

    Returns a dict with x, logits (list of 4), lam (list of 4) and, for proxy
    workloads, w_down [C_proxy][C] and w_up [C][C_proxy]; all in the
    workload's storage dtype.
    """
    device = torch.device(device)
    g = _gen(wl.seed if seed is None else seed, device)
    dt = wl.torch_dtype

    def randn(shape, scale=1.0):
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        if scale != 1.0:
            t.mul_(scale)
        return t.to(dt) if dt != torch.float32 else t

    def rand(shape):
        t = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
        return t.to(dt) if dt != torch.float32 else t

    out = {"x": randn((wl.n, wl.c, wl.h, wl.w))}
    logits, lams = [], []
    for d in range(4):
        S, L = wl.frame(d)
        logits.append(randn((wl.n, wl.cw, 3, S, L)))
        lams.append(rand((wl.n, wl.c_scan, S, L)))
    out["logits"] = logits
    out["lam"] = lams
    if wl.c_proxy > 0:
        out["w_down"] = randn((wl.c_proxy, wl.c), 1.0 / math.sqrt(wl.c))
        out["w_up"] = randn((wl.c, wl.c_proxy), 1.0 / math.sqrt(wl.c_proxy))
    return out


def constant_inputs(wl: Workload, x_value: float, lam_value: float = 1.0,
                    device="cpu", seed: int = 0) -> dict:
    """Constant x and lambda with random logits (used by the closed-form
    checks: with lambda = 1 and x = c, a scan's h at step t is (t+1) c)."""
    inp = make_inputs(wl, device, seed)
    inp["x"] = torch.full_like(inp["x"], x_value)
    inp["lam"] = [torch.full_like(l, lam_value) for l in inp["lam"]]
    return inp
