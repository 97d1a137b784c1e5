"""The forward as one launch (MOE_FFN_FP8_LAUNCH_SINGLE) against the oracle and against
the three-kernel launch, bit for bit: the phases run the same arithmetic in the same
order.  Each case runs the single launch several times in a row and between forwards of
the other mode, so that the phase counters (which only grow, one launch's count at a time)
are checked too; every debug forward also checks that no wait gave up (sync_timeouts)."""
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


def same(a, b):
    for k in KEYS:
        assert np.array_equal(np.asarray(a[k]).view(np.uint8), np.asarray(b[k]).view(np.uint8)), k


# hidden 5120 (the single launch's size); dense and routed, 1 to 8 tokens
@pytest.mark.parametrize("seed,M,E", [(71, 1, 0), (72, 4, 0), (73, 1, 8), (74, 3, 8), (75, 4, 8), (76, 5, 8),
                                      (77, 8, 8)])
def test_single_launch_matches_oracle_and_three_kernels(lib, seed, M, E):
    say("case single launch", seed, M, E)
    pr = Problem(seed, M, 5120, 512, E)
    ref = pr.run_oracle()
    three = pr.run_gpu()
    pr.ffn.set_launch_mode(F.LAUNCH_SINGLE)
    for rep in range(3):
        single = pr.run_gpu()
        same(single, three)
    check_all(single, ref, E, pr.weights)
    pr.ffn.set_launch_mode(F.LAUNCH_THREE)
    same(pr.run_gpu(), three)
    pr.ffn.set_launch_mode(F.LAUNCH_SINGLE)
    same(pr.run_gpu(), three)


def test_single_launch_consecutive_inputs(lib):
    """Consecutive single launches on different tokens and routes: each phase must read
    what the previous phase of the same launch stored, never a line an earlier launch
    left in a cache (the phases hand their data on with device-scope stores and loads)."""
    M, K, I, E = 4, 5120, 512, 8
    pr = Problem(78, M, K, I, E, force=[0, 1, 2, 3])
    x2 = W.activations(79, M, K, "cpu").to("cuda")
    l2 = W.router_logits(79, M, E, "cpu", force=[7, 6, 5, 5]).to("cuda")
    cases = [(pr.x, pr.logits), (x2, l2)]
    three = [pr.run_gpu(x=x, logits=lg) for x, lg in cases]
    assert not np.array_equal(three[0]["out"], three[1]["out"])
    pr.ffn.set_launch_mode(F.LAUNCH_SINGLE)
    for rep in range(6):
        x, lg = cases[rep % 2]
        same(pr.run_gpu(x=x, logits=lg), three[rep % 2])


def test_single_launch_full_size(lib):
    """The headline step's shape: hidden 5120, intermediate 8192, 128 routed experts + the
    shared one, 4 tokens on 4 distinct experts."""
    M, K, I, E = 4, W.HIDDEN, W.INTER, 128
    say("case single launch full size")
    pr = Problem(5, M, K, I, E, force=[3, 40, 77, 127])
    three = pr.run_gpu()
    pr.ffn.set_launch_mode(F.LAUNCH_SINGLE)
    single = pr.run_gpu()
    same(single, three)
    check_all(single, pr.run_oracle(), E, pr.weights)


def test_single_launch_graph_replays(lib):
    """Captured into a HIP graph, the single launch replays to the eager result (its
    launch count lives in device memory, advanced by its own last block, so every replay
    waits for its own phases)."""
    M = 4
    pr = Problem(8, M, 5120, 512, 6)
    pr.ffn.set_launch_mode(F.LAUNCH_SINGLE)
    out = torch.empty((M, 5120), dtype=torch.bfloat16, device="cuda")
    pr.ffn.forward(pr.x, pr.logits, out)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            pr.ffn.forward(pr.x, pr.logits, out)
    torch.cuda.synchronize()
    for i in range(5):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        pr.ffn.forward(pr.x, pr.logits, torch.empty_like(out))  # eager work in between


def test_single_launch_availability(lib):
    """SINGLE needs hidden 5120 and at most 8 tokens per launch; other modes are refused."""
    ok = F.MoeFFN(5120, 256, 2, 8)
    ok.set_launch_mode(F.LAUNCH_SINGLE)
    ok.set_launch_mode(F.LAUNCH_THREE)
    with pytest.raises(F.MoeError):
        ok.set_launch_mode(2)
    with pytest.raises(F.MoeError):
        F.MoeFFN(4096, 256, 2, 4).set_launch_mode(F.LAUNCH_SINGLE)
    with pytest.raises(F.MoeError):
        F.MoeFFN(5120, 256, 2, 16).set_launch_mode(F.LAUNCH_SINGLE)


@pytest.mark.parametrize("variant", [dict(gate_on_input=1), dict(x_scale=0.004, a_scale=0.02)],
                         ids=["gate_on_input", "static_scales"])
def test_single_launch_variant_readings(lib, variant):
    """The variant readings in the single launch: the three-kernel result bit for bit, and
    the oracle's variant to the parity bar."""
    M, K, I, E = 4, 5120, 512, 8
    pr = Problem(81, M, K, I, E)
    say("case single launch variant", variant)
    three = pr.run_gpu(variant=variant)
    pr.ffn.set_launch_mode(F.LAUNCH_SINGLE)
    for rep in range(2):
        same(pr.run_gpu(variant=variant), three)
    check_all(three, pr.run_oracle(variant=variant), E, pr.weights,
              gate_on_input=bool(variant.get("gate_on_input")), a_scale=variant.get("a_scale"))
