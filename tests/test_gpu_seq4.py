"""GPU parity of the plane-sequential four-direction kernel (seq4_kernel):
for many big planes (at least 256 (n, c) planes, sides multiples of 64 up to
1024) one workgroup per plane runs L2R, R2L, T2B and B2T in turn and builds
y in place, the horizontal directions reading x through LDS column tiles.
A last round of planes at most half full (one plane per CU) goes to the
concurrent four-direction path instead.  Every element is compared with the
fp64 oracle (normwise, 1e-5 for fp32 storage, 2e-2 for bf16), and the call
must report that kernel.  A forward keeping its states takes the same
kernel, which writes the fp32 scans bit for bit as the four-direction launch
does."""
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


# a forward keeping its states: the kernel also writes the four unweighted
# fp32 scans
STATE_CASES = [CASES[0], CASES[2], CASES[3], CASES[5], CASES[6]]


@pytest.mark.parametrize("chunk", [0, 7])
@pytest.mark.parametrize("shape,dtype,shared", STATE_CASES)
def test_seq4_keeps_states(shape, dtype, shared, chunk):
    """A forward keeping its states runs the plane-sequential kernel too (the
    tail's planes, if any, on the concurrent path into the same maps), with
    and without merge weights: y matches the oracle and agrees with the
    forward without states, each map matches the oracle's unweighted scan,
    the maps are the same bits with and without merge weights and as the
    four-direction launch's on the same planes (a forward over the first 64
    channels alone), and a backward from them returns the gradients of the
    recomputing backward (bit for bit, except channel-shared logits' sums
    in fp32 atomics)."""
    n, c, h, w = shape
    wl = Workload("case", n, c, h, w, dtype, shared, chunk, 1700 + h + w + c)
    print("seq4 states %s %s shared=%s chunk=%d" % (shape, dtype, shared, chunk), flush=True)
    sys.stdout.flush()
    inp = make_inputs(wl, DEV)
    ws = G.forward4_workspace(inp["x"], wl.cw)
    gm = torch.Generator(device=DEV)
    gm.manual_seed(11)
    m = torch.randn((4, c), generator=gm, device=DEV)
    st = G.states_buffer(inp["x"])
    y, times = G.gspn_forward4_timed(inp["x"], inp["logits"], inp["lam"], chunk_len=chunk, workspace=ws, states=st)
    plain = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], chunk_len=chunk, workspace=ws)
    stm = G.states_buffer(inp["x"])
    ym, timesm = G.gspn_forward4_timed(inp["x"], inp["logits"], inp["lam"], chunk_len=chunk, workspace=ws,
                                       merge=m, states=stm)
    plainm = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], chunk_len=chunk, workspace=ws, merge=m)
    torch.cuda.synchronize()
    # the first 64 channels of every image alone: too few planes for the
    # kernel, so the four-direction launch writes their states
    cs = 64
    sub_x = inp["x"][:, :cs].contiguous()
    sub_z = [z if wl.cw == 1 else z[:, :cs].contiguous() for z in inp["logits"]]
    sub_l = [l[:, :cs].contiguous() for l in inp["lam"]]
    sts = G.states_buffer(sub_x)
    _, timess = G.gspn_forward4_timed(sub_x, sub_z, sub_l, chunk_len=chunk,
                                      workspace=G.forward4_workspace(sub_x, 1 if wl.cw == 1 else cs), states=sts)
    torch.cuda.synchronize()
    for t in (times, timesm):
        assert t["scan_kernel"] == "seq4_kernel", t["scan_kernel"]
        assert t["tail"]["launches"] == (1 if _tail_split(n, c, False) else 0), t
    assert timess["scan_kernel"] != "seq4_kernel", timess["scan_kernel"]
    assert torch.equal(st, stm)
    for d in range(4):
        assert torch.equal(G.state_map(st, d, shape)[:, :cs], G.state_map(sts, d, tuple(sub_x.shape))), d
    # with states the kernel fuses lambda x + h into one multiply-add (as the
    # four-direction launch does) and applies a merge weight to h, without
    # it rounds the product first and scales lambda x: y agrees to rounding
    ref = oracle.forward4(inp["x"], inp["logits"], inp["lam"], chunk=chunk)
    refm = oracle.forward4(inp["x"], inp["logits"], inp["lam"], chunk=chunk, merge=_np(m))
    assert oracle.normwise_error(_np(y), ref) <= TOL[dtype]
    assert oracle.normwise_error(_np(ym), refm) <= TOL[dtype]
    assert oracle.normwise_error(_np(y), _np(plain)) <= TOL[dtype]
    assert oracle.normwise_error(_np(ym), _np(plainm)) <= TOL[dtype]
    for d in range(4):
        got = _np(G.state_map(st, d, shape))
        want = oracle.scan(d, inp["x"], inp["logits"][d], inp["lam"][d], chunk)
        if d >= 2:
            want = want.transpose(0, 1, 3, 2)  # the horizontal directions' scan frame
        assert oracle.normwise_error(got, want) <= TOL[dtype], d
    g = torch.Generator(device=DEV)
    g.manual_seed(wl.seed + 7)
    gy = torch.randn((n, c, h, w), generator=g, device=DEV, dtype=torch.float32).to(wl.torch_dtype)
    for mm, sts in ((None, st), (m, stm)):
        a = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk_len=chunk, merge=mm, states=sts)
        b = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk_len=chunk, merge=mm)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0])
        for d in range(4):
            assert torch.equal(a[2][d], b[2][d]), d
            if shared:
                # sums over the channels in fp32 atomics, whose order varies
                # between calls, each with cancellation, then rounded to the
                # storage type: the states' equality is checked above, so
                # here only agreement to the parity tolerance
                err = oracle.normwise_error(_np(a[1][d]), _np(b[1][d]))
                assert err <= TOL[dtype], (d, err)
            else:
                assert torch.equal(a[1][d], b[1][d]), d
