"""The allocation-free forward (moe_ffn_fp8_forward_scratch) through the C ABI against
moe_ffn_fp8_forward on the same handle: the same kernels over the library's static scratch
instead of the handle's workspace, so the same output bit for bit.  Two calls in a row, the
second with fewer tokens (the scratch keeps what the first left); a graph capture of it
replayed between eager calls; and the size limits it refuses."""
import numpy as np
import pytest
import torch

import fp8_moe_ffn_amd as F
import workloads as W
from harness import Problem

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _both(pr, x, lg):
    M = x.shape[0]
    want = torch.empty((M, pr.K), dtype=torch.bfloat16, device="cuda")
    got = torch.full((M, pr.K), 7.0, dtype=torch.bfloat16, device="cuda")
    pr.ffn.forward(x, lg, want)
    pr.ffn.forward_scratch(x, lg, got)
    torch.cuda.synchronize()
    return W.bits(got), W.bits(want)


@pytest.mark.parametrize("M,K,I,E,M2", [(8, 1024, 2048, 6, 3), (4, 5120, 8192, 8, 2), (16, 256, 512, 0, 5)])
def test_scratch_forward_matches_forward(lib, M, K, I, E, M2):
    say("case scratch forward", M, K, I, E, "then", M2)
    pr = Problem(60 + M, M, K, I, E)
    got, want = _both(pr, pr.x, pr.logits)
    assert np.array_equal(got, want)
    # a second call with fewer tokens and other inputs: nothing of the first may leak in
    x2 = W.activations(61 + M, M2, K, "cpu").cuda()
    l2 = W.router_logits(61 + M, M2, E, "cpu").cuda() if E else None
    got2, want2 = _both(pr, x2, l2)
    assert np.array_equal(got2, want2)
    assert not np.array_equal(got2, got[:M2])


def test_scratch_forward_graph_replays(lib):
    M, K, I, E = 4, 512, 1024, 6
    pr = Problem(62, M, K, I, E)
    out = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    pr.ffn.forward(pr.x, pr.logits, out)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pr.ffn.forward_scratch(pr.x, pr.logits, out)
    torch.cuda.synchronize()
    other = Problem(63, 2, K, I, E)
    for i in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        other.ffn.forward_scratch(other.x, other.logits, torch.empty((2, K), dtype=torch.bfloat16, device="cuda"))
        torch.cuda.synchronize()


def test_scratch_forward_limits(lib):
    strm = torch.cuda.current_stream().cuda_stream
    L = F.load()
    # more tokens than one launch of the decode kernels
    pr = Problem(64, 20, 256, 512, 3)
    out = torch.empty((20, 256), dtype=torch.bfloat16, device="cuda")
    st = L.moe_ffn_fp8_forward_scratch(pr.x.data_ptr(), pr.logits.data_ptr(), pr.ffn.handle, out.data_ptr(), 20, strm)
    assert st == F.ERR_UNSUPPORTED
    st = L.moe_ffn_fp8_forward_scratch(pr.x.data_ptr(), pr.logits.data_ptr(), pr.ffn.handle, out.data_ptr(), 21, strm)
    assert st == F.ERR_INVALID_ARG  # above max_tokens
    st = L.moe_ffn_fp8_forward_scratch(pr.x.data_ptr(), pr.logits.data_ptr(), pr.ffn.handle, out.data_ptr(), 16, strm)
    assert st == F.OK
    # a workspace above the scratch: 16 tokens at hidden 5120, intermediate 32768 (10.5 MB of partial sums)
    big = F.MoeFFN(5120, 32768, 0, 16)
    x = torch.zeros((16, 5120), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(x)
    assert L.moe_ffn_fp8_forward_scratch(x.data_ptr(), None, big.handle, o.data_ptr(), 16, strm) == F.ERR_UNSUPPORTED
    assert L.moe_ffn_fp8_forward_scratch(None, None, None, None, 1, strm) == F.ERR_INVALID_ARG
    big.close()
    torch.cuda.synchronize()
