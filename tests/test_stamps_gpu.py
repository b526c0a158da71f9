"""The measurement build of the library (libgdr_stamps.so: the flow kernel with shader-clock counters
compiled in) computes bit for bit what libgdr.so computes, and its counters are ordered."""
import ctypes
import os

import numpy as np
import pytest
import torch

from _dev import problem_to_dev
from gated_delta_rule_63_amd import gdr, inputs

pytestmark = pytest.mark.gpu

STAMPS = os.path.join(os.path.dirname(gdr.library_path()), "libgdr_stamps.so")


def _run(p, d):
    o, ht = gdr.gdr_chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu"], p.scale, d["h0"])
    torch.cuda.synchronize()
    return o, ht


def test_measurement_build_matches_and_its_counters_are_ordered():
    assert os.path.exists(STAMPS), "libgdr_stamps.so is built beside libgdr.so"
    lengths = [1000, 64, 333]
    p = inputs.prefill(lengths=lengths, HV=4)
    d = problem_to_dev(p)
    o1, h1 = _run(p, d)
    try:
        gdr.use_library(STAMPS)
        L = gdr.lib()
        L.gdr_dbg_flow_target.argtypes = [ctypes.c_int, ctypes.c_int]
        L.gdr_dbg_flow_stamps.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        assert L.gdr_dbg_flow_target(0, 1) == 0
        o2, h2 = _run(p, d)
        st = np.zeros((2, 128, 8), dtype=np.uint64)
        wg = np.zeros((8, 32, 4), dtype=np.uint64)
        assert L.gdr_dbg_flow_stamps(ctypes.c_void_p(st.ctypes.data), ctypes.c_void_p(wg.ctypes.data)) == 0
    finally:
        gdr.use_library(None)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(h1, h2)
    nc = (lengths[0] + 63) // 64
    s = st.astype(np.int64)
    for role in (0, 1):
        b = s[role]
        # barrier stamps: before <= after for both phases, and each iteration ends after the previous one
        assert np.all(b[:nc, 1] >= b[:nc, 0]) and np.all(b[:nc, 3] >= b[:nc, 2]) and np.all(b[:nc, 2] >= b[:nc, 1])
        assert np.all(np.diff(b[:nc + 1, 3]) > 0)
    a = s[0]
    for it in range(1, nc):  # inside phase X of the state waves: products, then R and the solve, then the rest
        assert a[it - 1, 3] < a[it, 5] <= a[it, 6] <= a[it, 0]
    w = wg.astype(np.int64)
    for n in range(len(lengths)):
        for h in range(p.HV):
            assert w[n, h, 2] > w[n, h, 0] and w[n, h, 3] > w[n, h, 1]
