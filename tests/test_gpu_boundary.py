"""The C ABI's handle life cycle on the GPU: a handle made by the stacked prepack
(moe_ffn_fp8_prepack, every expert slot from [E+1]-stacked arrays in one call) computes
what a handle filled slot by slot computes, and create frees everything it allocated when
one of its device allocations fails (forced through its test hook, the environment
variable MOE_FFN_FP8_FAIL_ALLOC)."""
import ctypes
import os

import numpy as np
import pytest
import torch

import fp8_moe_ffn_amd as F
import workloads as W
from harness import Problem, check_all

pytestmark = pytest.mark.gpu

KEYS = ("out", "xq", "s_x", "expert", "gate", "aq_shared", "s_a_shared", "aq_routed", "s_a_routed")


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("M,K,I,E", [(4, 256, 512, 4), (3, 384, 640, 0), (20, 512, 256, 6)])
def test_stacked_prepack(lib, M, K, I, E):
    """moe_ffn_fp8_prepack from stacked arrays: the same packed weights as slot-by-slot
    prepacking (unpacked back bit for bit), the same forward bit for bit, and the oracle's
    result to the parity bar."""
    say("case stacked prepack", M, K, I, E)
    pr = Problem(80 + M, M, K, I, E)
    experts = [W.Expert(*(t.cuda() for t in (e.w13, e.s13, e.w2, e.s2)))
               for e in (W.expert(pr.seed, slot, K, I, pr.gen_device) for slot in range(E + 1))]
    stack = [torch.stack([getattr(e, f) for e in experts]).contiguous() for f in ("w13", "w2", "s13", "s2")]
    h = F.MoeFFN.prepacked(K, I, E, M, *stack)
    for slot in range(E + 1):
        back = [torch.empty_like(t) for t in (experts[slot].w13, experts[slot].s13, experts[slot].w2,
                                              experts[slot].s2)]
        h.unpack_expert(slot, *back)
        torch.cuda.synchronize()
        for a, b in zip((experts[slot].w13, experts[slot].s13, experts[slot].w2, experts[slot].s2), back):
            assert torch.equal(a, b), slot
    ref_handle = pr.ffn
    pr.ffn = h
    got = pr.run_gpu()
    pr.ffn = ref_handle
    want = pr.run_gpu()
    for k in KEYS:
        assert np.array_equal(np.asarray(got[k]).view(np.uint8), np.asarray(want[k]).view(np.uint8)), k
    check_all(got, pr.run_oracle(), E, pr.weights)
    h.close()


def _hip():
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemGetInfo.argtypes = [ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    return hip


def _free_bytes(hip):
    torch.cuda.synchronize()
    free, total = ctypes.c_size_t(), ctypes.c_size_t()
    assert hip.hipMemGetInfo(ctypes.byref(free), ctypes.byref(total)) == 0
    return free.value


def test_create_frees_everything_when_an_allocation_fails(lib, monkeypatch):
    """For every allocation create makes (packed weights of 4 Maverick-size experts,
    about 500 MB, the forward workspace and the grouped workspace), failing it returns
    MOE_FFN_FP8_ERR_OUT_OF_MEMORY, leaves *out NULL and leaves the device's free memory
    where it was; past the last allocation the same call succeeds.  The stacked prepack
    fails the same way."""
    hip = _hip()
    L = F.load()
    dims = F.Dims(W.HIDDEN, W.INTER, 3, 64)  # above 8 tokens: the grouped workspace too
    h = ctypes.c_void_p()
    assert L.moe_ffn_fp8_create(ctypes.byref(dims), ctypes.byref(h)) == F.OK  # first use of the kernels
    assert L.moe_ffn_fp8_destroy(h) == F.OK
    base = _free_bytes(hip)
    failures = 0
    for n in range(1, 64):
        monkeypatch.setenv("MOE_FFN_FP8_FAIL_ALLOC", str(n))
        h = ctypes.c_void_p(1234)
        st = L.moe_ffn_fp8_create(ctypes.byref(dims), ctypes.byref(h))
        if st == F.OK:
            assert h.value
            assert L.moe_ffn_fp8_destroy(h) == F.OK
            break
        assert st == F.ERR_OUT_OF_MEMORY, (n, st)
        assert h.value is None, n
        failures += 1
        leak = base - _free_bytes(hip)
        assert abs(leak) < (16 << 20), (n, leak)
    say("allocations failed one at a time:", failures)
    assert failures >= 20  # weights (4), forward workspace (7), grouped workspace (10)
    # the stacked prepack: create fails inside it
    small = F.Dims(256, 512, 2, 4)
    ex = [W.expert(1, s, 256, 512, "cuda") for s in range(3)]
    stack = [torch.stack([getattr(e, f) for e in ex]).contiguous() for f in ("w13", "w2", "s13", "s2")]
    base = _free_bytes(hip)  # after torch's own allocations for the inputs
    monkeypatch.setenv("MOE_FFN_FP8_FAIL_ALLOC", "3")
    h = ctypes.c_void_p(1234)
    st = L.moe_ffn_fp8_prepack(ctypes.byref(small), *(t.data_ptr() for t in stack),
                               torch.cuda.current_stream().cuda_stream, ctypes.byref(h))
    assert st == F.ERR_OUT_OF_MEMORY and h.value is None
    monkeypatch.delenv("MOE_FFN_FP8_FAIL_ALLOC")
    leak = base - _free_bytes(hip)
    assert abs(leak) < (16 << 20), leak
