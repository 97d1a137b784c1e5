"""The grouped pass's item order (fp8_moe_ffn_amd/csrc/group_order.hpp), built for the host:
a bijection that spreads the shared expert's items over the fixed share and keeps them out
of the pool."""

import ctypes
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("group") / "libgroup_host.so")
    src = os.path.join(ROOT, "tests", "csrc", "group_host.cpp")
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-D__host__=", "-D__device__=",
           "-I", os.path.join(ROOT, "fp8_moe_ffn_amd", "csrc"), src, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    lib = ctypes.CDLL(out)
    lib.host_group_order.restype = None
    return lib


def order(lib, ns, total, G):
    out = np.zeros(total, np.int32)
    lib.host_group_order(ns, total, G, out.ctypes.data_as(ctypes.c_void_p))
    return out, lib.host_group_fixed_share(total, G)


# (shared items, slots, blocks): I/16 pairs of FC13 or (K/64) * nsplit tiles of FC2, 1 + d slots
@pytest.mark.parametrize("ns,slots,G", [(512, 62, 256), (640, 62, 256), (512, 1, 256), (32, 5, 32),
                                        (512, 2, 256), (64, 200, 64), (128, 3, 128), (80, 7, 80)])
def test_group_order(lib, ns, slots, G):
    total = ns * slots
    m, F = order(lib, ns, total, G)
    assert sorted(m.tolist()) == list(range(total)), "not a bijection"
    shared_at = np.nonzero(m < ns)[0]
    assert (m[shared_at] == np.arange(ns)).all(), "shared items out of order"
    assert shared_at.max() < max(F, ns), "a shared item in the pool"
    if slots > 1 and F > ns:
        gaps = np.diff(shared_at)
        assert gaps.min() >= F // ns and gaps.max() <= -(-F // ns), "shared items not evenly spread"
    routed = m[m >= ns]
    assert (np.diff(routed) == 1).all(), "routed items out of slot-major order"
    assert (m[F:] == np.arange(F, total)).all() if F < total else True
