"""Thin ctypes binding of libgspn (include/gspn.h).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in libgspn's HIP kernels.
The functions carry the C ABI's names.  Shapes, dtypes, devices and
contiguity are checked here so that the pointers handed to the library
always cover the sizes it is told; everything else (and the error codes) is
the library's.

If libgspn.so is missing, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# GSPN_LIBRARY may point the binding at another build of libgspn.
LIB_PATH = os.environ.get("GSPN_LIBRARY") or os.path.join(_PKG, "libgspn.so")

T2B, B2T, L2R, R2L = 0, 1, 2, 3
DIRECTIONS = ("T2B", "B2T", "L2R", "R2L")
GSPN_F32, GSPN_BF16 = 0, 1

STATUS = {
    0: "GSPN_OK", 1: "GSPN_ERR_NULL_POINTER", 2: "GSPN_ERR_BAD_SHAPE", 3: "GSPN_ERR_BAD_DIRECTION",
    4: "GSPN_ERR_BAD_DTYPE", 5: "GSPN_ERR_BAD_CHUNK", 6: "GSPN_ERR_BAD_WEIGHT_CHANNELS",
    7: "GSPN_ERR_MISALIGNED", 8: "GSPN_ERR_ALIASING", 9: "GSPN_ERR_UNSUPPORTED", 10: "GSPN_ERR_HIP",
    11: "GSPN_ERR_WORKSPACE", 12: "GSPN_ERR_BAD_LAYOUT",
}

# gspn_layout: where the per-direction logits / lambdas live.
LAYOUTS = {"scan": 0, "array": 1}

# Symbols declared in include/gspn.h.
EXPORTS = ("gspn_normalize_weights", "gspn_scan_fwd", "gspn_merge4", "gspn_proxy_project",
           "gspn_scan4_fwd", "gspn_forward4_workspace_bytes", "gspn_forward4",
           "gspn_proxy_forward4_workspace_bytes", "gspn_proxy_forward4", "gspn_forward4_timed",
           "gspn_proxy_forward4_timed", "gspn_backward4_workspace_bytes", "gspn_backward4", "gspn_backward4_timed",
           "gspn_forward4_noalloc", "gspn_proxy_backward4_workspace_bytes", "gspn_proxy_backward4",
           "gspn_proxy_backward4_timed", "gspn_proxy_states_bytes", "gspn_status_string", "gspn_abi_version")

# GSPN_NOALLOC_SCRATCH_BYTES: the static scratch gspn_forward4_noalloc works in.
NOALLOC_SCRATCH_BYTES = 64 << 20

# gspn_stage, in order.
STAGES = ("project_down", "normalize", "transpose", "scan", "combine", "project_up", "adjoint", "reduce", "layout",
          "tail", "weight_grad")


# gspn_scan_kernel, in order.
SCAN_KERNELS = ("none", "scan_kernel", "scan4v_kernel", "scan4lp_kernel", "plane4_kernel", "scan4band_kernel",
                "seq4_kernel")


class AdjointPlan(ctypes.Structure):
    _fields_ = [("family", ctypes.c_int32), ("positions_per_lane", ctypes.c_int32),
                ("channel_group", ctypes.c_int32), ("nontemporal", ctypes.c_int32)]


# gspn_adjoint_plan.family, in order.
ADJOINT_FAMILIES = ("none", "adj4_kernel", "adjplane_kernel", "adj4band_kernel")


class StageTimes(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_float * len(STAGES)), ("launches", ctypes.c_int32 * len(STAGES)),
                ("scan_kernel", ctypes.c_int32), ("adjoint", AdjointPlan)]

    def as_dict(self) -> dict:
        d = {name: {"ms": float(self.ms[i]), "launches": int(self.launches[i])}
             for i, name in enumerate(STAGES)}
        d["scan_kernel"] = SCAN_KERNELS[self.scan_kernel]
        a = self.adjoint
        d["adjoint_plan"] = {"kernel": ADJOINT_FAMILIES[a.family], "positions_per_lane": int(a.positions_per_lane),
                             "channel_group": int(a.channel_group), "nontemporal": bool(a.nontemporal)}
        return d


class GspnError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__("%s failed: %s" % (call, lib().gspn_status_string(status).decode()))


_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libgspn with argument types set.  Raises if it is not built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    "libgspn.so is not built (expected at %s); run "
                    "`python -m linear_spatial_propagation_gspn_amd.build`" % LIB_PATH)
            h = ctypes.CDLL(LIB_PATH)
            i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
            h.gspn_normalize_weights.argtypes = [ci, i64, i64, i64, i64, vp, vp, ci, vp]
            h.gspn_scan_fwd.argtypes = [ci, i64, i64, i64, i64, i64, i64, vp, vp, ci, vp, vp, ci, ci, vp]
            h.gspn_merge4.argtypes = [vp, vp, vp, vp, vp, i64, ci, vp]
            h.gspn_proxy_project.argtypes = [i64, i64, i64, i64, i64, vp, vp, vp, ci, vp]
            h.gspn_scan4_fwd.argtypes = [i64, i64, i64, i64, i64, i64, vp, ctypes.POINTER(vp),
                                         ctypes.POINTER(vp), ctypes.POINTER(vp), ci, vp]
            h.gspn_scan4_fwd.restype = ci
            h.gspn_forward4_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, ci, ci]
            h.gspn_forward4_workspace_bytes.restype = i64
            h.gspn_proxy_forward4_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, ci, ci]
            h.gspn_proxy_forward4_workspace_bytes.restype = i64
            h.gspn_proxy_forward4.argtypes = [i64, i64, i64, i64, i64, i64, i64, vp, vp, vp,
                                              ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, vp, vp, i64, ci, ci,
                                              vp]
            h.gspn_proxy_states_bytes.argtypes = [i64, i64, i64, i64, ci]
            h.gspn_proxy_states_bytes.restype = i64
            h.gspn_proxy_forward4.restype = ci
            h.gspn_forward4.argtypes = [i64, i64, i64, i64, i64, i64, vp, ctypes.POINTER(vp),
                                        ctypes.POINTER(vp), vp, vp, vp, vp, i64, ci, ci, vp]
            h.gspn_forward4_noalloc.argtypes = [i64, i64, i64, i64, i64, i64, vp, ctypes.POINTER(vp),
                                                ctypes.POINTER(vp), vp, vp, vp, ci, ci, vp]
            h.gspn_forward4_noalloc.restype = ci
            h.gspn_forward4_timed.argtypes = h.gspn_forward4.argtypes + [ctypes.POINTER(StageTimes)]
            h.gspn_forward4_timed.restype = ci
            h.gspn_proxy_forward4_timed.argtypes = h.gspn_proxy_forward4.argtypes + [ctypes.POINTER(StageTimes)]
            h.gspn_proxy_forward4_timed.restype = ci
            for name in ("gspn_normalize_weights", "gspn_scan_fwd", "gspn_merge4",
                         "gspn_proxy_project", "gspn_forward4"):
                getattr(h, name).restype = ci
            h.gspn_backward4_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, ci, ci]
            h.gspn_backward4_workspace_bytes.restype = i64
            h.gspn_backward4.argtypes = [i64, i64, i64, i64, i64, i64, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp,
                                         vp, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), vp, vp, i64, ci, ci, vp]
            h.gspn_backward4.restype = ci
            h.gspn_backward4_timed.argtypes = h.gspn_backward4.argtypes + [ctypes.POINTER(StageTimes)]
            h.gspn_backward4_timed.restype = ci
            h.gspn_proxy_backward4_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, ci, ci]
            h.gspn_proxy_backward4_workspace_bytes.restype = i64
            h.gspn_proxy_backward4.argtypes = [i64, i64, i64, i64, i64, i64, i64, vp, vp, vp, ctypes.POINTER(vp),
                                               ctypes.POINTER(vp), vp, vp, vp, vp, vp, vp, ctypes.POINTER(vp),
                                               ctypes.POINTER(vp), vp, vp, i64, ci, ci, vp]
            h.gspn_proxy_backward4.restype = ci
            h.gspn_proxy_backward4_timed.argtypes = h.gspn_proxy_backward4.argtypes + [ctypes.POINTER(StageTimes)]
            h.gspn_proxy_backward4_timed.restype = ci
            h.gspn_status_string.argtypes = [ci]
            h.gspn_status_string.restype = ctypes.c_char_p
            h.gspn_abi_version.argtypes = []
            h.gspn_abi_version.restype = ci
            _lib = h
        return _lib


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GSPN_F32
    if t.dtype == torch.bfloat16:
        return GSPN_BF16
    raise TypeError("libgspn stores float32 or bfloat16, got %s" % t.dtype)


def _check(t: torch.Tensor, name: str, shape: tuple, dtype: torch.dtype, device) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.device != device or t.device.type != "cuda":
        raise ValueError("%s must live on %s (a HIP device)" % (name, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _raise(st: int, call: str) -> None:
    if st != 0:
        raise GspnError(st, call)


def frame_shape(direction: int, h: int, w: int) -> tuple[int, int]:
    """(S, L): scan steps and line length of a direction."""
    return (w, h) if direction in (L2R, R2L) else (h, w)


def _layout_code(layout: str) -> int:
    if layout not in LAYOUTS:
        raise ValueError("layout must be one of %s, got %r" % (tuple(LAYOUTS), layout))
    return LAYOUTS[layout]


def tensor_frame(direction: int, h: int, w: int, layout: str = "scan") -> tuple[int, int]:
    """(rows, cols) of a direction's logit / lambda planes in ``layout``:
    its scan frame (S, L) for "scan", (H, W) for "array"."""
    _layout_code(layout)
    return (h, w) if layout == "array" else frame_shape(direction, h, w)


def to_scan_frame(t: torch.Tensor, direction: int) -> torch.Tensor:
    """An [..., H, W] tensor in the scan frame of ``direction`` (contiguous
    copy of the transpose for the horizontal directions)."""
    return t.transpose(-1, -2).contiguous() if direction in (L2R, R2L) else t.contiguous()


def gspn_normalize_weights(direction: int, logits: torch.Tensor, h: int, w: int,
                           out: torch.Tensor | None = None) -> torch.Tensor:
    """Sigmoid + row normalisation of one direction's logits [N][Cw][3][S][L]."""
    n, cw = logits.shape[0], logits.shape[1]
    S, L = frame_shape(direction, h, w)
    _check(logits, "logits", (n, cw, 3, S, L), logits.dtype, logits.device)
    if out is None:
        out = torch.empty_like(logits)
    _check(out, "out", logits.shape, logits.dtype, logits.device)
    _raise(lib().gspn_normalize_weights(direction, n, cw, h, w, _ptr(logits), _ptr(out),
                                        _dtype_code(logits), _stream(logits.device)),
           "gspn_normalize_weights")
    return out


def gspn_scan_fwd(direction: int, x: torch.Tensor, wts: torch.Tensor, lam: torch.Tensor,
                  chunk_len: int = 0, wts_are_logits: bool = True,
                  out: torch.Tensor | None = None, accumulate: bool = False) -> torch.Tensor:
    """One direction of the line scan.  x [N][C][H][W]; wts [N][Cw][3][S][L];
    lam [N][C][S][L]; returns out (= h, or out += h when accumulate)."""
    n, c, h, w = x.shape
    S, L = frame_shape(direction, h, w)
    dt = x.dtype
    cw = wts.shape[1] if wts.dim() == 5 else -1
    _check(x, "x", (n, c, h, w), dt, x.device)
    _check(wts, "wts", (n, cw, 3, S, L), dt, x.device)
    _check(lam, "lam", (n, c, S, L), dt, x.device)
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an out tensor")
        out = torch.empty_like(x)
    _check(out, "out", (n, c, h, w), dt, x.device)
    _raise(lib().gspn_scan_fwd(direction, int(chunk_len), n, c, h, w, cw, _ptr(x), _ptr(wts),
                               1 if wts_are_logits else 0, _ptr(lam), _ptr(out),
                               1 if accumulate else 0, _dtype_code(x), _stream(x.device)),
           "gspn_scan_fwd")
    return out


def gspn_merge4(hs: Sequence[torch.Tensor], out: torch.Tensor | None = None) -> torch.Tensor:
    """y = h0 + h1 + h2 + h3 elementwise."""
    h0 = hs[0]
    _dtype_code(h0)
    for i, t in enumerate(hs):
        _check(t, "h%d" % i, h0.shape, h0.dtype, h0.device)
    if out is None:
        out = torch.empty_like(h0)
    _check(out, "out", h0.shape, h0.dtype, h0.device)
    _raise(lib().gspn_merge4(_ptr(hs[0]), _ptr(hs[1]), _ptr(hs[2]), _ptr(hs[3]), _ptr(out),
                             h0.numel(), _dtype_code(h0), _stream(h0.device)), "gspn_merge4")
    return out


def gspn_proxy_project(inp: torch.Tensor, weight: torch.Tensor,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """1x1 projection: out[n, o] = sum_c weight[o, c] inp[n, c] per pixel."""
    n, cin, h, w = inp.shape
    cout = weight.shape[0]
    _check(inp, "inp", (n, cin, h, w), inp.dtype, inp.device)
    _check(weight, "weight", (cout, cin), inp.dtype, inp.device)
    if out is None:
        out = torch.empty((n, cout, h, w), dtype=inp.dtype, device=inp.device)
    _check(out, "out", (n, cout, h, w), inp.dtype, inp.device)
    _raise(lib().gspn_proxy_project(n, cin, h, w, cout, _ptr(inp), _ptr(weight), _ptr(out),
                                    _dtype_code(inp), _stream(inp.device)), "gspn_proxy_project")
    return out


def gspn_scan4_fwd(x: torch.Tensor, logits: Sequence[torch.Tensor], lams: Sequence[torch.Tensor],
                   chunk_len: int = 0, outs: Sequence[torch.Tensor] | None = None) -> list:
    """The four directions' scans in one launch, each into its own output."""
    n, c, h, w = x.shape
    dt = x.dtype
    cw = logits[0].shape[1]
    _check(x, "x", (n, c, h, w), dt, x.device)
    for d in range(4):
        S, L = frame_shape(d, h, w)
        _check(logits[d], "logits[%d]" % d, (n, cw, 3, S, L), dt, x.device)
        _check(lams[d], "lam[%d]" % d, (n, c, S, L), dt, x.device)
    if outs is None:
        outs = [torch.empty_like(x) for _ in range(4)]
    for d in range(4):
        _check(outs[d], "out[%d]" % d, (n, c, h, w), dt, x.device)
    zp = (ctypes.c_void_p * 4)(*[z.data_ptr() for z in logits])
    lp = (ctypes.c_void_p * 4)(*[l.data_ptr() for l in lams])
    op = (ctypes.c_void_p * 4)(*[o.data_ptr() for o in outs])
    _raise(lib().gspn_scan4_fwd(n, c, h, w, cw, int(chunk_len), _ptr(x), zp, lp, op, _dtype_code(x),
                                _stream(x.device)), "gspn_scan4_fwd")
    return list(outs)


def gspn_forward4_workspace_bytes(x: torch.Tensor, cw: int, layout: str = "scan") -> int:
    """Bytes of the optional gspn_forward4 workspace for inputs shaped like x
    with cw weight channels (1 = channel-shared)."""
    n, c, h, w = x.shape
    return int(lib().gspn_forward4_workspace_bytes(n, c, h, w, cw, _dtype_code(x), _layout_code(layout)))


def forward4_workspace(x: torch.Tensor, cw: int, layout: str = "scan") -> torch.Tensor:
    """A workspace buffer (uint8 tensor on x's device) for gspn_forward4."""
    nbytes = gspn_forward4_workspace_bytes(x, cw, layout)
    if nbytes < 0:
        raise ValueError("invalid shape for a gspn_forward4 workspace")
    return torch.empty(nbytes, dtype=torch.uint8, device=x.device)


def _merge_ptr(merge, c: int, device, name: str = "merge"):
    """The device pointer of fp32 merge weights [4][c] (None: the plain sum)."""
    if merge is None:
        return None
    _check(merge, name, (4, c), torch.float32, device)
    return _ptr(merge)


def states_buffer(x: torch.Tensor) -> torch.Tensor:
    """A buffer for the four directions' fp32 forward states of inputs shaped
    like x (see gspn_forward4's ``states``)."""
    return torch.empty(4 * x.numel(), dtype=torch.float32, device=x.device)


def state_map(states: torch.Tensor, d: int, x_shape: tuple) -> torch.Tensor:
    """Direction d's map in a states buffer: [N][C][S_d][L_d] in its scan
    frame ([N][C][H][W] for T2B / B2T, [N][C][W][H] for L2R / R2L)."""
    n, c, h, w = x_shape
    S, L = frame_shape(d, h, w)
    e = n * c * h * w
    return states.view(-1)[d * e:(d + 1) * e].view(n, c, S, L)


def _states_ptr(states, x):
    if states is None:
        return None
    _check(states, "states", (4 * x.numel(),), torch.float32, x.device)
    return _ptr(states)


def _forward4(x, logits, lams, chunk_len, out, workspace, times, merge=None, states=None, layout="scan"):
    n, c, h, w = x.shape
    dt = x.dtype
    cw = logits[0].shape[1]
    lc = _layout_code(layout)
    _check(x, "x", (n, c, h, w), dt, x.device)
    for d in range(4):
        S, L = tensor_frame(d, h, w, layout)
        _check(logits[d], "logits[%d]" % d, (n, cw, 3, S, L), dt, x.device)
        _check(lams[d], "lam[%d]" % d, (n, c, S, L), dt, x.device)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", (n, c, h, w), dt, x.device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        if workspace.device != x.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on %s" % x.device)
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel() * workspace.element_size()
    zp = (ctypes.c_void_p * 4)(*[z.data_ptr() for z in logits])
    lp = (ctypes.c_void_p * 4)(*[l.data_ptr() for l in lams])
    mp = _merge_ptr(merge, c, x.device)
    sp = _states_ptr(states, x)
    args = (n, c, h, w, cw, int(chunk_len), _ptr(x), zp, lp, mp, _ptr(out), sp, ws_ptr, ws_bytes, _dtype_code(x),
            lc, _stream(x.device))
    if times is None:
        _raise(lib().gspn_forward4(*args), "gspn_forward4")
    else:
        _raise(lib().gspn_forward4_timed(*args, ctypes.byref(times)), "gspn_forward4_timed")
    return out


def gspn_forward4(x: torch.Tensor, logits: Sequence[torch.Tensor], lams: Sequence[torch.Tensor],
                  chunk_len: int = 0, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, merge: torch.Tensor | None = None,
                  states: torch.Tensor | bool | None = None, layout: str = "scan"):
    """Four-direction propagation; logits[d] / lams[d] in direction d's scan
    frame (layout "scan") or all in the array frame [.., H, W] (layout
    "array", which needs the workspace).  The directions are summed, or with
    ``merge`` (fp32 [4][C] on the device) weighted per direction and channel.
    ``workspace`` (see forward4_workspace) lets the library run the four
    directions concurrently when that pays.  ``states`` (True, or a buffer
    from states_buffer) also keeps the four directions' fp32 scans for
    gspn_backward4 (needs the workspace); the call then returns (out,
    states)."""
    if states is True:
        states = states_buffer(x)
    if states is None or states is False:
        return _forward4(x, logits, lams, chunk_len, out, workspace, None, merge, layout=layout)
    return _forward4(x, logits, lams, chunk_len, out, workspace, None, merge, states, layout), states


def gspn_forward4_noalloc(x: torch.Tensor, logits: Sequence[torch.Tensor], lams: Sequence[torch.Tensor],
                          chunk_len: int = 0, out: torch.Tensor | None = None, merge: torch.Tensor | None = None,
                          states: torch.Tensor | None = None, layout: str = "scan") -> torch.Tensor:
    """gspn_forward4 without a workspace argument: the library works in its
    static per-GPU scratch array (NOALLOC_SCRATCH_BYTES), so the call
    allocates nothing on the device (``out`` and ``states``, if given, are the
    caller's).  Calls that overlap in time on one GPU race on that array."""
    n, c, h, w = x.shape
    dt = x.dtype
    cw = logits[0].shape[1]
    lc = _layout_code(layout)
    _check(x, "x", (n, c, h, w), dt, x.device)
    for d in range(4):
        S, L = tensor_frame(d, h, w, layout)
        _check(logits[d], "logits[%d]" % d, (n, cw, 3, S, L), dt, x.device)
        _check(lams[d], "lam[%d]" % d, (n, c, S, L), dt, x.device)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", (n, c, h, w), dt, x.device)
    zp = (ctypes.c_void_p * 4)(*[z.data_ptr() for z in logits])
    lp = (ctypes.c_void_p * 4)(*[l.data_ptr() for l in lams])
    _raise(lib().gspn_forward4_noalloc(n, c, h, w, cw, int(chunk_len), _ptr(x), zp, lp,
                                       _merge_ptr(merge, c, x.device), _ptr(out), _states_ptr(states, x),
                                       _dtype_code(x), lc, _stream(x.device)), "gspn_forward4_noalloc")
    return out


def gspn_forward4_timed(x: torch.Tensor, logits: Sequence[torch.Tensor], lams: Sequence[torch.Tensor],
                        chunk_len: int = 0, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None,
                        merge: torch.Tensor | None = None,
                        states: torch.Tensor | None = None, layout: str = "scan") -> tuple[torch.Tensor, dict]:
    """gspn_forward4 with HIP events around every launch; returns (out,
    {stage: {"ms", "launches"}}).  Waits for the stream to reach its end."""
    times = StageTimes()
    out = _forward4(x, logits, lams, chunk_len, out, workspace, times, merge, states, layout)
    return out, times.as_dict()


def proxy_forward4_workspace(x: torch.Tensor, c_proxy: int, cw: int, layout: str = "scan") -> torch.Tensor:
    """A workspace buffer (uint8 tensor on x's device) for gspn_proxy_forward4."""
    n, c, h, w = x.shape
    nbytes = int(lib().gspn_proxy_forward4_workspace_bytes(n, c, h, w, c_proxy, cw, _dtype_code(x),
                                                           _layout_code(layout)))
    if nbytes < 0:
        raise ValueError("invalid shape for a gspn_proxy_forward4 workspace")
    return torch.empty(nbytes, dtype=torch.uint8, device=x.device)


def proxy_states_buffer(x: torch.Tensor, c_proxy: int) -> torch.Tensor:
    """A buffer (uint8 tensor on x's device, 256-byte aligned) for the
    proxy-space state gspn_proxy_forward4 keeps for gspn_proxy_backward4."""
    n, c, h, w = x.shape
    nbytes = int(lib().gspn_proxy_states_bytes(n, c_proxy, h, w, _dtype_code(x)))
    if nbytes < 0:
        raise ValueError("invalid shape for a proxy states buffer")
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=x.device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + nbytes]


def _proxy_forward4(x, w_down, w_up, logits, lams, chunk_len, out, workspace, times, merge=None, layout="scan",
                    states=None):
    n, c, h, w = x.shape
    dt = x.dtype
    cp = w_down.shape[0]
    cw = logits[0].shape[1]
    lc = _layout_code(layout)
    _check(x, "x", (n, c, h, w), dt, x.device)
    _check(w_down, "w_down", (cp, c), dt, x.device)
    _check(w_up, "w_up", (c, cp), dt, x.device)
    for d in range(4):
        S, L = tensor_frame(d, h, w, layout)
        _check(logits[d], "logits[%d]" % d, (n, cw, 3, S, L), dt, x.device)
        _check(lams[d], "lam[%d]" % d, (n, cp, S, L), dt, x.device)
    if out is None:
        out = torch.empty_like(x)
    _check(out, "out", (n, c, h, w), dt, x.device)
    if workspace is None:
        workspace = proxy_forward4_workspace(x, cp, cw, layout)
    if workspace.device != x.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % x.device)
    zp = (ctypes.c_void_p * 4)(*[z.data_ptr() for z in logits])
    lp = (ctypes.c_void_p * 4)(*[l.data_ptr() for l in lams])
    mp = _merge_ptr(merge, cp, x.device)
    sp = None
    if states is not None:
        if states.device != x.device or not states.is_contiguous():
            raise ValueError("states must be a contiguous buffer on %s" % x.device)
        if states.numel() * states.element_size() < lib().gspn_proxy_states_bytes(n, cp, h, w, _dtype_code(x)):
            raise ValueError("states buffer too small (see proxy_states_buffer)")
        sp = _ptr(states)
    args = (n, c, h, w, cp, cw, int(chunk_len), _ptr(x), _ptr(w_down), _ptr(w_up), zp, lp, mp, _ptr(out), sp,
            _ptr(workspace), workspace.numel() * workspace.element_size(), _dtype_code(x), lc, _stream(x.device))
    if times is None:
        _raise(lib().gspn_proxy_forward4(*args), "gspn_proxy_forward4")
    else:
        _raise(lib().gspn_proxy_forward4_timed(*args, ctypes.byref(times)), "gspn_proxy_forward4_timed")
    return out


def gspn_proxy_forward4(x: torch.Tensor, w_down: torch.Tensor, w_up: torch.Tensor,
                        logits: Sequence[torch.Tensor], lams: Sequence[torch.Tensor],
                        chunk_len: int = 0, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, merge: torch.Tensor | None = None,
                        layout: str = "scan", states: torch.Tensor | bool | None = None):
    """Compressive-proxy forward: C -> C_proxy 1x1 projection, four-direction
    scan in proxy space (summed, or weighted by ``merge`` fp32 [4][C_proxy]),
    C_proxy -> C projection.  ``states`` (True, or a buffer from
    proxy_states_buffer) also keeps x_p, y_p and the proxy-space fp32 scans
    for gspn_proxy_backward4; the call then returns (out, states)."""
    if states is True:
        states = proxy_states_buffer(x, w_down.shape[0])
    if states is None or states is False:
        return _proxy_forward4(x, w_down, w_up, logits, lams, chunk_len, out, workspace, None, merge, layout)
    return _proxy_forward4(x, w_down, w_up, logits, lams, chunk_len, out, workspace, None, merge, layout,
                           states), states


def gspn_proxy_forward4_timed(x: torch.Tensor, w_down: torch.Tensor, w_up: torch.Tensor,
                              logits: Sequence[torch.Tensor], lams: Sequence[torch.Tensor],
                              chunk_len: int = 0, out: torch.Tensor | None = None,
                              workspace: torch.Tensor | None = None,
                              merge: torch.Tensor | None = None, layout: str = "scan",
                              states: torch.Tensor | None = None) -> tuple[torch.Tensor, dict]:
    """gspn_proxy_forward4 with HIP events around every launch; returns (out,
    {stage: {"ms", "launches"}}); ``states``: a buffer to keep the proxy-space
    state in, as for gspn_proxy_forward4."""
    times = StageTimes()
    out = _proxy_forward4(x, w_down, w_up, logits, lams, chunk_len, out, workspace, times, merge, layout, states)
    return out, times.as_dict()


def backward4_workspace(x: torch.Tensor, cw: int, with_states: bool = False, layout: str = "scan") -> torch.Tensor:
    """A workspace buffer (uint8 tensor on x's device) for gspn_backward4;
    with_states: for calls given the forward states (16 * x.numel() bytes
    smaller)."""
    n, c, h, w = x.shape
    nbytes = int(lib().gspn_backward4_workspace_bytes(n, c, h, w, cw, _dtype_code(x), _layout_code(layout)))
    if nbytes < 0:
        raise ValueError("invalid shape for a gspn_backward4 workspace")
    if with_states:
        nbytes -= 16 * x.numel()
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)


def gspn_backward4(x: torch.Tensor, logits: Sequence[torch.Tensor], lams: Sequence[torch.Tensor],
                   gy: torch.Tensor, chunk_len: int = 0, workspace: torch.Tensor | None = None,
                   out: tuple | None = None, times: StageTimes | None = None,
                   merge: torch.Tensor | None = None, dmerge: torch.Tensor | bool | None = None,
                   states: torch.Tensor | None = None, layout: str = "scan") -> tuple:
    """Gradients of gspn_forward4 (with the same ``merge``) for dL/dy = gy:
    returns (dx, [dlogits_d], [dlam_d]) in the inputs' layouts, and also the
    merge weights' gradient (fp32 [4][C]) as a fourth element when ``merge``
    is given or ``dmerge`` is (a tensor to fill, or True).  ``out`` may
    supply the first three; ``times`` (a StageTimes) selects
    gspn_backward4_timed and receives the stage durations; ``states`` (from
    gspn_forward4) spares the recompute of the forward; ``layout`` as in
    gspn_forward4 (the gradients come in the same layout as the inputs)."""
    n, c, h, w = x.shape
    dt = x.dtype
    cw = logits[0].shape[1]
    lc = _layout_code(layout)
    _check(x, "x", (n, c, h, w), dt, x.device)
    _check(gy, "gy", (n, c, h, w), dt, x.device)
    for d in range(4):
        S, L = tensor_frame(d, h, w, layout)
        _check(logits[d], "logits[%d]" % d, (n, cw, 3, S, L), dt, x.device)
        _check(lams[d], "lam[%d]" % d, (n, c, S, L), dt, x.device)
    if out is None:
        dx = torch.empty_like(x)
        dz = [torch.empty_like(z) for z in logits]
        dl = [torch.empty_like(l) for l in lams]
    else:
        dx, dz, dl = out
    _check(dx, "dx", (n, c, h, w), dt, x.device)
    for d in range(4):
        _check(dz[d], "dlogits[%d]" % d, tuple(logits[d].shape), dt, x.device)
        _check(dl[d], "dlam[%d]" % d, tuple(lams[d].shape), dt, x.device)
    want_dm = merge is not None or (dmerge is not None and dmerge is not False)
    if want_dm and not isinstance(dmerge, torch.Tensor):
        dmerge = torch.empty((4, c), dtype=torch.float32, device=x.device)
    mp = _merge_ptr(merge, c, x.device)
    dmp = _merge_ptr(dmerge, c, x.device, "dmerge") if want_dm else None
    sp = _states_ptr(states, x)
    if workspace is None:
        workspace = backward4_workspace(x, cw, with_states=states is not None, layout=layout)
    if workspace.device != x.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % x.device)
    vp4 = ctypes.c_void_p * 4
    args = (n, c, h, w, cw, int(chunk_len), _ptr(x), vp4(*[z.data_ptr() for z in logits]),
            vp4(*[l.data_ptr() for l in lams]), mp, sp, _ptr(gy), _ptr(dx), vp4(*[t.data_ptr() for t in dz]),
            vp4(*[t.data_ptr() for t in dl]), dmp, _ptr(workspace), workspace.numel() * workspace.element_size(),
            _dtype_code(x), lc, _stream(x.device))
    if times is None:
        _raise(lib().gspn_backward4(*args), "gspn_backward4")
    else:
        _raise(lib().gspn_backward4_timed(*args, ctypes.byref(times)), "gspn_backward4_timed")
    return (dx, dz, dl, dmerge) if want_dm else (dx, dz, dl)


def proxy_backward4_workspace(x: torch.Tensor, c_proxy: int, cw: int, layout: str = "scan") -> torch.Tensor:
    """A workspace buffer (uint8 tensor on x's device) for gspn_proxy_backward4."""
    n, c, h, w = x.shape
    nbytes = int(lib().gspn_proxy_backward4_workspace_bytes(n, c, h, w, c_proxy, cw, _dtype_code(x),
                                                            _layout_code(layout)))
    if nbytes < 0:
        raise ValueError("invalid shape for a gspn_proxy_backward4 workspace")
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)


def gspn_proxy_backward4(x: torch.Tensor, w_down: torch.Tensor, w_up: torch.Tensor,
                         logits: Sequence[torch.Tensor], lams: Sequence[torch.Tensor], gy: torch.Tensor,
                         chunk_len: int = 0, workspace: torch.Tensor | None = None,
                         times: StageTimes | None = None, merge: torch.Tensor | None = None,
                         dmerge: torch.Tensor | bool | None = None, layout: str = "scan",
                         states: torch.Tensor | None = None) -> tuple:
    """Gradients of gspn_proxy_forward4 (with the same ``merge``) for dL/dy =
    gy: returns (dx, dw_down fp32 [C_proxy][C], dw_up fp32 [C][C_proxy],
    [dlogits_d], [dlam_d]) and, when ``merge`` is given or ``dmerge`` is (a
    tensor to fill, or True), the merge weights' gradient (fp32
    [4][C_proxy]) last.  ``times`` (a StageTimes) selects
    gspn_proxy_backward4_timed; ``layout`` as in gspn_proxy_forward4;
    ``states`` (what gspn_proxy_forward4 kept for the same inputs) spares the
    recompute of x_p and of the proxy-space forward."""
    n, c, h, w = x.shape
    dt = x.dtype
    cp = w_down.shape[0]
    cw = logits[0].shape[1]
    lc = _layout_code(layout)
    _check(x, "x", (n, c, h, w), dt, x.device)
    _check(gy, "gy", (n, c, h, w), dt, x.device)
    _check(w_down, "w_down", (cp, c), dt, x.device)
    _check(w_up, "w_up", (c, cp), dt, x.device)
    for d in range(4):
        S, L = tensor_frame(d, h, w, layout)
        _check(logits[d], "logits[%d]" % d, (n, cw, 3, S, L), dt, x.device)
        _check(lams[d], "lam[%d]" % d, (n, cp, S, L), dt, x.device)
    dx = torch.empty_like(x)
    dwd = torch.empty((cp, c), dtype=torch.float32, device=x.device)
    dwu = torch.empty((c, cp), dtype=torch.float32, device=x.device)
    dz = [torch.empty_like(z) for z in logits]
    dl = [torch.empty_like(l) for l in lams]
    want_dm = merge is not None or (dmerge is not None and dmerge is not False)
    if want_dm and not isinstance(dmerge, torch.Tensor):
        dmerge = torch.empty((4, cp), dtype=torch.float32, device=x.device)
    mp = _merge_ptr(merge, cp, x.device)
    dmp = _merge_ptr(dmerge, cp, x.device, "dmerge") if want_dm else None
    if workspace is None:
        workspace = proxy_backward4_workspace(x, cp, cw, layout)
    if workspace.device != x.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % x.device)
    sp = None
    if states is not None:
        if states.device != x.device or not states.is_contiguous():
            raise ValueError("states must be a contiguous buffer on %s" % x.device)
        if states.numel() * states.element_size() < lib().gspn_proxy_states_bytes(n, cp, h, w, _dtype_code(x)):
            raise ValueError("states buffer too small (see proxy_states_buffer)")
        sp = _ptr(states)
    vp4 = ctypes.c_void_p * 4
    args = (n, c, h, w, cp, cw, int(chunk_len), _ptr(x), _ptr(w_down), _ptr(w_up),
            vp4(*[z.data_ptr() for z in logits]), vp4(*[l.data_ptr() for l in lams]), mp, sp, _ptr(gy), _ptr(dx),
            _ptr(dwd), _ptr(dwu), vp4(*[t.data_ptr() for t in dz]), vp4(*[t.data_ptr() for t in dl]), dmp,
            _ptr(workspace), workspace.numel() * workspace.element_size(), _dtype_code(x), lc, _stream(x.device))
    if times is None:
        _raise(lib().gspn_proxy_backward4(*args), "gspn_proxy_backward4")
    else:
        _raise(lib().gspn_proxy_backward4_timed(*args, ctypes.byref(times)), "gspn_proxy_backward4_timed")
    res = (dx, dwd, dwu, dz, dl)
    return res + (dmerge,) if want_dm else res


class _Forward4(torch.autograd.Function):
    """gspn_forward4 as an autograd node whose backward is gspn_backward4."""

    @staticmethod
    def forward(ctx, chunk_len, has_merge, keep, x, merge, *tensors):
        logits, lams = list(tensors[:4]), list(tensors[4:])
        cw = logits[0].shape[1]
        m = merge if has_merge else None
        states = states_buffer(x) if keep else torch.empty(0, device=x.device)
        y = gspn_forward4(x, logits, lams, chunk_len=chunk_len, workspace=forward4_workspace(x, cw), merge=m,
                          states=states if keep else None)
        if keep:
            y = y[0]
        ctx.chunk_len = chunk_len
        ctx.has_merge = has_merge
        ctx.keep = keep
        ctx.save_for_backward(x, merge, states, *tensors)
        return y

    @staticmethod
    def backward(ctx, gy):
        x, merge, states, *tensors = ctx.saved_tensors
        logits, lams = tensors[:4], tensors[4:]
        res = gspn_backward4(x, logits, lams, gy.to(x.dtype).contiguous(), chunk_len=ctx.chunk_len,
                             merge=merge if ctx.has_merge else None, states=states if ctx.keep else None)
        dx, dz, dl = res[0], res[1], res[2]
        dm = res[3] if ctx.has_merge else None
        return (None, None, None, dx, dm, *dz, *dl)


def gspn4(x: torch.Tensor, logits: Sequence[torch.Tensor], lams: Sequence[torch.Tensor], chunk_len: int = 0,
          merge: torch.Tensor | None = None, keep_states: bool = False) -> torch.Tensor:
    """The four-direction propagation as a differentiable op: gspn_forward4
    forward, gspn_backward4 for the gradients of x, the logits, the lambdas
    and (if given) the merge weights.  keep_states: the forward keeps its
    fp32 scans (16 bytes per element of x, held until the backward) so the
    backward need not recompute them; only for planes larger than 64 x 64
    (for smaller ones the one-pass forward and the plane-resident backward,
    which recomputes the states inside its launch, are faster than keeping
    them)."""
    has_merge = merge is not None
    m = merge if has_merge else torch.empty(0, device=x.device)
    h, w = x.shape[-2:]
    keep = bool(keep_states) and (h > 64 or w > 64)
    return _Forward4.apply(int(chunk_len), has_merge, keep, x, m, *logits, *lams)


class _ProxyForward4(torch.autograd.Function):
    """gspn_proxy_forward4 as an autograd node whose backward is
    gspn_proxy_backward4 (weight gradients cast to the weights' dtype)."""

    @staticmethod
    def forward(ctx, chunk_len, has_merge, keep, x, w_down, w_up, merge, *tensors):
        logits, lams = list(tensors[:4]), list(tensors[4:])
        states = proxy_states_buffer(x, w_down.shape[0]) if keep else torch.empty(0, device=x.device)
        y = gspn_proxy_forward4(x, w_down, w_up, logits, lams, chunk_len=chunk_len,
                                merge=merge if has_merge else None, states=states if keep else None)
        if keep:
            y = y[0]
        ctx.chunk_len = chunk_len
        ctx.has_merge = has_merge
        ctx.keep = keep
        ctx.save_for_backward(x, w_down, w_up, merge, states, *tensors)
        return y

    @staticmethod
    def backward(ctx, gy):
        x, w_down, w_up, merge, states, *tensors = ctx.saved_tensors
        logits, lams = tensors[:4], tensors[4:]
        res = gspn_proxy_backward4(x, w_down, w_up, logits, lams, gy.to(x.dtype).contiguous(),
                                   chunk_len=ctx.chunk_len, merge=merge if ctx.has_merge else None,
                                   states=states if ctx.keep else None)
        dx, dwd, dwu, dz, dl = res[:5]
        dm = res[5] if ctx.has_merge else None
        return (None, None, None, dx, dwd.to(w_down.dtype), dwu.to(w_up.dtype), dm, *dz, *dl)


def gspn_proxy4(x: torch.Tensor, w_down: torch.Tensor, w_up: torch.Tensor, logits: Sequence[torch.Tensor],
                lams: Sequence[torch.Tensor], chunk_len: int = 0, merge: torch.Tensor | None = None,
                keep_states: bool = False) -> torch.Tensor:
    """The compressive-proxy propagation as a differentiable op:
    gspn_proxy_forward4 forward, gspn_proxy_backward4 for the gradients of
    x, both projection weights, the logits, the lambdas and (if given) the
    merge weights.  keep_states: the forward keeps x_p, y_p and the
    proxy-space fp32 scans (gspn_proxy_states_bytes, held until the
    backward) so the backward recomputes none of them."""
    has_merge = merge is not None
    m = merge if has_merge else torch.empty(0, device=x.device)
    return _ProxyForward4.apply(int(chunk_len), has_merge, bool(keep_states), x, w_down, w_up, m, *logits, *lams)
