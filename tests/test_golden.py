"""Regression snapshot of the seeded tiny workload (inputs and oracle output)."""
import json
import os

import numpy as np

import oracle
from linear_spatial_propagation_gspn_amd.workloads import WORKLOADS, make_inputs

HERE = os.path.dirname(os.path.abspath(__file__))


def _load():
    with open(os.path.join(HERE, "golden", "tiny_forward4.json")) as f:
        return json.load(f)


def test_seeded_generator_reproduces_stored_inputs():
    rec = _load()
    inp = make_inputs(WORKLOADS["tiny"], "cpu")
    assert inp["x"].flatten().tolist() == rec["x"]
    for d in range(4):
        assert inp["logits"][d].flatten().tolist() == rec["logits"][d]
        assert inp["lam"][d].flatten().tolist() == rec["lam"][d]


def test_oracle_reproduces_stored_outputs():
    rec = _load()
    wl = WORKLOADS["tiny"]
    shape = (wl.n, wl.c, wl.h, wl.w)
    x = np.array(rec["x"]).reshape(shape)
    zs = [np.array(z).reshape((wl.n, wl.cw, 3) + wl.frame(d)) for d, z in enumerate(rec["logits"])]
    ls = [np.array(l).reshape((wl.n, wl.c) + wl.frame(d)) for d, l in enumerate(rec["lam"])]
    for chunk in (0, 8):
        ref = np.array([float.fromhex(v) for v in rec["y_chunk%d" % chunk]]).reshape(shape)
        got = oracle.forward4(x, zs, ls, chunk=chunk)
        np.testing.assert_allclose(got, ref, rtol=1e-14, atol=1e-14)
