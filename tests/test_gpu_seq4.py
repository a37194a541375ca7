"""GPU parity of the plane-sequential four-direction kernel (seq4_kernel):
for many big planes (at least 256 (n, c) planes, sides multiples of 64 up to
1024) one workgroup per plane runs L2R, R2L, T2B and B2T in turn and builds
y in place, the horizontal directions reading x through LDS column tiles.
A last round of planes at most half full (one plane per CU) goes to the
concurrent four-direction path instead.  Every element is compared with the
fp64 oracle (normwise, 1e-5 for fp32 storage, 2e-2 for bf16), and the call
must report that kernel."""
import sys

import pytest
import torch

import oracle
from linear_spatial_propagation_gspn_amd import gspn as G
from linear_spatial_propagation_gspn_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
DEV = "cuda"


def _np(t):
    return t.detach().float().cpu().double().numpy()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    yield
    torch.cuda.synchronize()


CASES = [
    # (n, c, h, w), storage, channel-shared logits
    ((1, 256, 64, 128), "bf16", True),    # half-pair weights, lines of 64 and 128 positions
    ((2, 130, 128, 64), "bf16", True),    # 260 planes over two images
    ((1, 256, 128, 192), "bf16", False),  # per-channel bf16 logits normalised in the scan
    ((2, 128, 128, 64), "f32", False),    # per-channel fp32 logits
    ((1, 256, 192, 128), "f32", True),    # shared fp32 logits over 256 channels (fp32 weight triples)
    ((1, 300, 64, 128), "bf16", True),    # 256 + 44 planes: the last 44 on the concurrent path
    ((2, 150, 64, 128), "f32", False),    # the same for per-channel logits, the 44 in the second image
]

CUS = 256  # compute units of the MI355X


def _tail_split(n, c, merge):
    planes = n * c
    tail = planes % CUS
    return planes > CUS and 0 < tail and 2 * tail <= CUS and (planes - tail) // c == (planes - 1) // c


@pytest.mark.parametrize("merge", [False, True])
@pytest.mark.parametrize("chunk", [0, 7, 64])
@pytest.mark.parametrize("shape,dtype,shared", CASES)
def test_seq4_matches_oracle(shape, dtype, shared, chunk, merge):
    n, c, h, w = shape
    wl = Workload("case", n, c, h, w, dtype, shared, chunk, 1300 + h + w + c)
    print("seq4 %s %s shared=%s chunk=%d merge=%s" % (shape, dtype, shared, chunk, merge), flush=True)
    sys.stdout.flush()
    inp = make_inputs(wl, DEV)
    m = None
    if merge:
        g = torch.Generator(device=DEV)
        g.manual_seed(7)
        m = torch.randn((4, c), generator=g, device=DEV)
    y, times = G.gspn_forward4_timed(inp["x"], inp["logits"], inp["lam"], chunk_len=chunk,
                                     workspace=G.forward4_workspace(inp["x"], wl.cw), merge=m)
    torch.cuda.synchronize()
    assert times["scan_kernel"] == "seq4_kernel", times["scan_kernel"]
    # a last round of planes at most half full runs on the concurrent path,
    # timed as one stage
    assert times["transpose"]["launches"] == 0 and times["combine"]["launches"] == 0, times
    assert times["scan"]["launches"] == 1
    assert times["tail"]["launches"] == (1 if _tail_split(n, c, merge) else 0), times
    ref = oracle.forward4(inp["x"], inp["logits"], inp["lam"], chunk=chunk, merge=None if m is None else _np(m))
    assert oracle.normwise_error(_np(y), ref) <= TOL[dtype]


def test_seq4_deterministic():
    wl = Workload("case", 1, 256, 64, 128, "bf16", True, 0, 5)
    inp = make_inputs(wl, DEV)
    ws = G.forward4_workspace(inp["x"], wl.cw)
    a = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], workspace=ws)
    b = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("c", [256, 300])   # 300: the last 44 planes on the concurrent path
def test_seq4_array_layout_and_noalloc(c):
    """The array layout (horizontal tensors copied into their scan frame
    first) and the allocation-free entry point reach the same kernel and the
    same bits."""
    wl = Workload("case", 1, c, 64, 128, "bf16", True, 0, 6)
    inp = make_inputs(wl, DEV)
    ys = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], workspace=G.forward4_workspace(inp["x"], wl.cw))
    za = [z if d < 2 else z.transpose(-1, -2).contiguous() for d, z in enumerate(inp["logits"])]
    la = [l if d < 2 else l.transpose(-1, -2).contiguous() for d, l in enumerate(inp["lam"])]
    ya, times = G.gspn_forward4_timed(inp["x"], za, la, workspace=G.forward4_workspace(inp["x"], wl.cw, "array"),
                                      layout="array")
    yn = G.gspn_forward4_noalloc(inp["x"], inp["logits"], inp["lam"])
    torch.cuda.synchronize()
    assert times["scan_kernel"] == "seq4_kernel"
    assert times["tail"]["launches"] == (1 if _tail_split(1, c, False) else 0)
    assert torch.equal(ya, ys) and torch.equal(yn, ys)
