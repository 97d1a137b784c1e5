"""Pins for ``oracle.ffn`` against things other than the oracle itself.

* exactness of the float64 contraction, checked with int64 arithmetic;
* the loop-only implementation ``oracle.loops`` (different algorithms) on the
  tiny configuration;
* a worked example whose every number is derived by hand below;
* torch's silu; the fused versus unfused FC13;
* algebraic invariants (powers of two through the scales, batching, relabelling
  experts, zero rows, special routings).
"""

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import ffn, fp8, loops


def problem(seed, m, hidden, inter, num_experts, force=None):
    x = W.bits(W.activations(seed, m, hidden))
    lg = W.bits(W.router_logits(seed, m, num_experts, force=force)) if num_experts else None
    experts = [W.expert(seed, f, hidden, inter).numpy() for f in range(num_experts + 1)]
    return x, lg, experts


def test_contraction_is_exact_int64():
    rng = np.random.default_rng(0)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    hidden = 5120
    xq = rng.choice(finite, size=(4, hidden))
    w = rng.choice(finite, size=(hidden, 64))
    w[:, 0] = 0x7E  # worst case magnitude: 448 * 448 * K
    xq[0, :] = 0x7E
    units = lambda c: np.rint(fp8.e4m3_decode(c) * 512).astype(np.int64)  # exact: multiples of 2**-9
    exact = units(xq) @ units(w)  # int64, in units of 2**-18
    got = fp8.e4m3_decode(xq) @ fp8.e4m3_decode(w)
    assert np.array_equal(got * 2.0 ** 18, exact.astype(np.float64))
    assert np.all(np.abs(exact) < 2 ** 53)


def test_tiny_config_matches_loop_only_version():
    c = W.TINY
    x, lg, experts = problem(c["seed"], c["M"], c["hidden"], c["inter"], c["num_experts"])
    r = ffn.forward(x, lg, experts, c["num_experts"])

    def lw(slot):
        e = experts[slot]
        return e.w13.tolist(), e.s13.astype(np.float64).tolist(), e.w2.tolist(), e.s2.astype(np.float64).tolist()

    ref = loops.forward(x.tolist(), lg.tolist(), lw, c["num_experts"])
    assert np.array_equal(r["xq"], np.array(ref["xq"], np.uint8))
    assert np.array_equal(r["s_x"], np.array(ref["s_x"]))
    assert r["expert"].tolist() == ref["expert"]
    np.testing.assert_allclose(r["gate"], ref["gate"], rtol=1e-15)
    assert np.array_equal(r["aq_shared"], np.array(ref["aq_shared"], np.uint8))
    np.testing.assert_allclose(r["s_a_shared"], ref["s_a_shared"], rtol=1e-15)
    assert np.array_equal(r["aq_routed"], np.array(ref["aq_routed"], np.uint8))
    np.testing.assert_allclose(r["s_a_routed"], ref["s_a_routed"], rtol=1e-15)
    np.testing.assert_allclose(r["ref"], np.array(ref["ref"]), rtol=1e-12, atol=1e-300)
    assert np.array_equal(r["out"], np.array(ref["out"], np.uint16))
    # the step is not degenerate: several experts are used and outputs are O(1)
    assert len(set(r["expert"].tolist())) >= 2
    assert 1e-3 < np.sqrt(np.mean(r["ref"] ** 2)) < 1e3


def test_worked_example_by_hand():
    """K = 4, I = 2, one token, dense.  Every number below is derived by hand.

    x = [7, 0, 0, 0]  ->  amax 7, s_x = 7/448 = 2**-6 exactly, xq[0] = e4m3(448) = 0x7E.
    W13 row 0 = [1.0 (0x38), -0.5 (0xB0) | 2.0 (0x40), 0.25 (0x28)], other rows 1.0.
    s13 = [2**-2, 1, 1, 1].  Only k = 0 contributes, acc = 448 * w, h = 7 * w * s13:
        g = [1.75, -3.5],  u = [14, 1.75]
        a0 = 1.75 * sigmoid(1.75) * 14,  a1 = -3.5 * sigmoid(-3.5) * 1.75
    s_a = fp32(a0 / 448); a0 / s_a rounds to 0x7E; a1 / s_a = -3.8535...,
    whose nearest e4m3 values are 3.75 (0x47) and 4.0: 3.75 is nearer -> 0xC7.
    W2 = all 1.0 (0x38), s2 = [1, 2, 0.5, 1]:
        y[k] = (448 - 3.75) * s_a * s2[k] = 444.25 * s_a * s2[k].
    Swapping gate and up would give a1 / a0 = silu(1.75) ... a different code.
    """
    x = np.array([[0x40E0, 0, 0, 0]], np.uint16)  # bf16 7.0
    w13 = np.full((4, 4), 0x38, np.uint8)
    w13[0] = [0x38, 0xB0, 0x40, 0x28]
    s13 = np.array([0.25, 1, 1, 1], np.float32)
    w2 = np.full((2, 4), 0x38, np.uint8)
    s2 = np.array([1, 2, 0.5, 1], np.float32)
    r = ffn.forward(x, None, [ffn.ExpertWeights(w13, s13, w2, s2)], 0)
    assert r["s_x"][0] == 2.0 ** -6
    assert r["xq"][0].tolist() == [0x7E, 0, 0, 0]
    sig = lambda z: 1 / (1 + math.exp(-z))
    a0 = 1.75 * sig(1.75) * 14
    a1 = -3.5 * sig(-3.5) * 1.75
    np.testing.assert_allclose(r["a_shared"][0], [a0, a1], rtol=1e-15)
    s_a = float(np.float32(a0 / 448))
    assert r["s_a_shared"][0] == s_a
    assert r["aq_shared"][0].tolist() == [0x7E, 0xC7]
    np.testing.assert_allclose(r["ref"][0], [444.25 * s_a * v for v in (1, 2, 0.5, 1)], rtol=1e-15)


def test_routing_ties_and_gate():
    lg = np.array([[1.0, 3.0, 3.0, 2.0], [0.0, -1.0, 0.0, 0.0], [-5.0, -6.0, -7.0, -4.0]])
    e, gate = ffn.route_top1(lg)
    assert e.tolist() == [1, 0, 3]  # lowest index among equal maxima
    assert gate[1] == 0.5  # sigmoid(0) exactly
    np.testing.assert_allclose(gate, [1 / (1 + math.exp(-3)), 0.5, 1 / (1 + math.exp(4))], rtol=1e-15)


def test_swiglu_against_torch_and_fused_vs_unfused():
    x, _, experts = problem(3, 3, 256, 128, 0)
    w = experts[0]
    xq, s_x = ffn.quantize_rows(fp8.bf16_to_f64(x))
    a = ffn.fc13_swiglu(xq, s_x, w)
    h1 = ffn.linear_fp8(xq, s_x, w.w13[:, :128], w.s13[:128])
    h3 = ffn.linear_fp8(xq, s_x, w.w13[:, 128:], w.s13[128:])
    h = ffn.linear_fp8(xq, s_x, w.w13, w.s13)
    assert np.array_equal(h, np.concatenate([h1, h3], axis=1))
    ref = (torch.nn.functional.silu(torch.from_numpy(h1)) * torch.from_numpy(h3)).numpy()
    np.testing.assert_allclose(a, ref, rtol=1e-14, atol=0)
    assert ffn.swiglu(np.array([0.0]), np.array([5.0]))[0] == 0.0
    assert ffn.swiglu(np.array([-1e4]), np.array([5.0]))[0] == 0.0
    np.testing.assert_allclose(ffn.swiglu(np.array([60.0]), np.array([2.0])), [120.0], rtol=1e-15)


@pytest.mark.parametrize("j", [3, -2])
def test_power_of_two_scale_invariants(j):
    x, _, experts = problem(5, 2, 256, 128, 0)
    base = ffn.forward(x, None, experts, 0)
    e = experts[0]
    up = ffn.ExpertWeights(e.w13, e.s13.copy(), e.w2, e.s2)
    up.s13[128:] *= np.float32(2.0 ** j)  # up projection scaled: a, s_a, y scale, codes don't
    r = ffn.forward(x, None, [up], 0)
    assert np.array_equal(r["aq_shared"], base["aq_shared"])
    assert np.array_equal(r["s_a_shared"], base["s_a_shared"] * 2.0 ** j)
    assert np.array_equal(r["ref"], base["ref"] * 2.0 ** j)
    down = ffn.ExpertWeights(e.w13, e.s13, e.w2, e.s2 * np.float32(2.0 ** j))
    r = ffn.forward(x, None, [down], 0)
    assert np.array_equal(r["ref"], base["ref"] * 2.0 ** j)


def test_batching_rows_are_independent():
    x, lg, experts = problem(1, 4, 256, 128, 4)
    full = ffn.forward(x, lg, experts, 4)
    for m in range(4):
        one = ffn.forward(x[m:m + 1], lg[m:m + 1], experts, 4)
        assert np.array_equal(one["out"][0], full["out"][m])
        assert np.array_equal(one["ref"][0], full["ref"][m])
        assert np.array_equal(one["aq_routed"][0], full["aq_routed"][m])


def test_relabelling_experts_changes_nothing():
    x, lg, experts = problem(2, 4, 256, 128, 4)
    perm = [2, 0, 3, 1]
    new = [None] * 5
    for e in range(4):
        new[perm[e]] = experts[e]
    new[4] = experts[4]
    lg2 = np.zeros_like(lg)
    for e in range(4):
        lg2[:, perm[e]] = lg[:, e]
    a = ffn.forward(x, lg, experts, 4)
    b = ffn.forward(x, lg2, new, 4)
    vals = fp8.bf16_to_f64(lg)
    assert all((vals[m] == vals[m].max()).sum() == 1 for m in range(4))  # no ties here
    assert np.array_equal(a["out"], b["out"])
    assert [perm[e] for e in a["expert"]] == b["expert"].tolist()


def test_all_tokens_one_expert_equals_two_dense_runs():
    x, lg, experts = problem(4, 4, 256, 128, 4, force=[2, 2, 2, 2])
    r = ffn.forward(x, lg, experts, 4)
    assert r["expert"].tolist() == [2, 2, 2, 2]
    sh = ffn.forward(x, None, [experts[4]], 0)["y_shared"]
    ro = ffn.forward(x, None, [experts[2]], 0)["y_shared"]
    assert np.array_equal(r["ref"], sh + r["gate"][:, None] * ro)


def test_zeroed_shared_or_routed_experts():
    x, lg, experts = problem(6, 3, 256, 128, 4)
    full = ffn.forward(x, lg, experts, 4)
    sh0 = list(experts)
    e = experts[4]
    sh0[4] = ffn.ExpertWeights(e.w13, np.zeros_like(e.s13), e.w2, e.s2)
    r = ffn.forward(x, lg, sh0, 4)
    assert np.array_equal(r["ref"], full["gate"][:, None] * full["y_routed"])
    ro0 = [ffn.ExpertWeights(f.w13, f.s13, f.w2, np.zeros_like(f.s2)) for f in experts[:4]] + [experts[4]]
    r = ffn.forward(x, lg, ro0, 4)
    assert np.array_equal(r["ref"], full["y_shared"])


def test_zero_token_row_and_empty_batch():
    x, lg, experts = problem(8, 3, 256, 128, 4)
    x = x.copy()
    x[1] = 0
    r = ffn.forward(x, lg, experts, 4)
    assert r["s_x"][1] == 0 and not r["xq"][1].any()
    assert r["s_a_shared"][1] == 0 and not r["aq_shared"][1].any()
    assert not r["ref"][1].any()
    e0 = ffn.forward(x[:0], lg[:0], experts, 4)
    assert e0["out"].shape == (0, 256)


def _loop_weights(experts):
    def lw(slot):
        e = experts[slot]
        return e.w13.tolist(), e.s13.astype(np.float64).tolist(), e.w2.tolist(), e.s2.astype(np.float64).tolist()
    return lw


@pytest.mark.parametrize("variant", [
    dict(gate_on_input=True),
    dict(x_scale="low"),
    dict(a_scale="low"),
    dict(x_scale="low", a_scale="low"),
    dict(gate_on_input=True, x_scale="low", a_scale="low"),
])
def test_variant_readings_match_loop_only_version(variant):
    """The variant readings (gate on the routed expert's input; static calibrated
    scales, chosen so that some codes saturate at 448) against the independent
    loop-only evaluation, bitwise."""
    seed, M, K, I, E = 11, 3, 128, 128, 2
    x, lg, experts = problem(seed, M, K, I, E)
    base = ffn.forward(x, lg, experts, E)
    v = dict(variant)
    if v.get("x_scale") == "low":  # half the smallest per-token scale: the largest |x| saturate
        v["x_scale"] = float(np.float32(base["s_x"].min() / 2))
    if v.get("a_scale") == "low":
        v["a_scale"] = float(np.float32(min(base["s_a_shared"].min(), base["s_a_routed"].min()) / 2))
    r = ffn.forward(x, lg, experts, E, **v)
    ref = loops.forward(x.tolist(), lg.tolist(), _loop_weights(experts), E, **v)
    assert np.array_equal(r["xq"], np.array(ref["xq"], np.uint8))
    assert np.array_equal(r["aq_shared"], np.array(ref["aq_shared"], np.uint8))
    assert np.array_equal(r["aq_routed"], np.array(ref["aq_routed"], np.uint8))
    np.testing.assert_allclose(r["s_a_routed"], ref["s_a_routed"], rtol=1e-15)
    np.testing.assert_allclose(r["ref"], np.array(ref["ref"]), rtol=1e-12, atol=1e-300)
    assert np.array_equal(r["out"], np.array(ref["out"], np.uint16))
    if "x_scale" in v:
        assert (r["xq"] & 0x7F == 0x7E).any() and (r["s_x"] == v["x_scale"]).all()
    if "a_scale" in v:
        assert (r["aq_shared"] & 0x7F == 0x7E).any()
    assert not np.array_equal(r["out"], base["out"])  # the variant changes the result


def test_static_scales_that_equal_the_dynamic_ones_change_nothing():
    """One token, dense: static x and intermediate scales equal to that token's
    dynamic scales give the dynamic result bit for bit."""
    x, _, experts = problem(5, 1, 256, 256, 0)
    dyn = ffn.forward(x, None, experts, 0)
    st = ffn.forward(x, None, experts, 0, x_scale=float(dyn["s_x"][0]), a_scale=float(dyn["s_a_shared"][0]))
    for k in ("xq", "aq_shared", "ref", "out"):
        assert np.array_equal(st[k], dyn[k]), k


def test_input_gate_of_one_is_the_output_gate():
    """A routed logit of 64 gives a gate of exactly 1 in float64; gating the input or
    the output then computes the same thing."""
    seed, M, K, I, E = 12, 4, 128, 256, 3
    x, lg, experts = problem(seed, M, K, I, E)
    lg = lg.copy()
    lg[:, 1] = 0x4280  # bf16 64.0 on expert 1 for every token
    out = ffn.forward(x, lg, experts, E)
    inp = ffn.forward(x, lg, experts, E, gate_on_input=True)
    assert (out["gate"] == 1.0).all() and (out["expert"] == 1).all()
    for k in ("aq_routed", "s_a_routed", "ref", "out"):
        assert np.array_equal(inp[k], out[k]), k


def test_static_quantisation_saturates():
    v = np.array([0.0, 1.0, -1.0, 447.0, 448.0, 449.0, 1e6, -1e6])
    c = ffn.quantize_static(v, 1.0)
    assert c.tolist() == [0x00, 0x38, 0xB8, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]
    assert ffn.quantize_static(v * 2.0 ** -5, 2.0 ** -5).tolist() == c.tolist()


def _norm_weight(seed, hidden):
    return W.bits(W.norm_weight(seed, hidden))


def test_rmsnorm_against_torch_and_its_invariants():
    h = fp8.bf16_to_f64(W.bits(W.activations(3, 5, 256)))
    w = fp8.bf16_to_f64(_norm_weight(3, 256))
    got = ffn.rmsnorm(h, w, 1e-5)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(h), (256,), torch.from_numpy(w), eps=1e-5).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=0)
    # without eps: invariant under a power-of-two scaling of h, bit for bit; unit RMS with w = 1
    assert np.array_equal(ffn.rmsnorm(h * 2.0 ** 7, w, 0.0), ffn.rmsnorm(h, w, 0.0))
    u = ffn.rmsnorm(h, np.ones(256), 0.0)
    np.testing.assert_allclose(np.mean(u * u, axis=1), 1.0, rtol=1e-14)
    # eps matters only against a small mean square
    z = np.zeros((1, 256)); z[0, 5] = 1e-4
    assert ffn.rmsnorm(z, np.ones(256), 1e-5)[0, 5] < ffn.rmsnorm(z, np.ones(256), 0.0)[0, 5]


@pytest.mark.parametrize("variant", [dict(), dict(gate_on_input=True, x_scale="low")])
def test_fused_rmsnorm_step_matches_loop_only_version(variant):
    seed, M, K, I, E = 13, 3, 128, 128, 2
    x, lg, experts = problem(seed, M, K, I, E)
    nw = _norm_weight(seed, K)
    base = ffn.forward(x, lg, experts, E, norm_w_bits=nw)
    v = dict(variant)
    if v.get("x_scale") == "low":
        v["x_scale"] = float(np.float32(base["s_x"].min() / 2))
    r = ffn.forward(x, lg, experts, E, norm_w_bits=nw, norm_eps=1e-5, **v)
    ref = loops.forward(x.tolist(), lg.tolist(), _loop_weights(experts), E, norm_w_bits=nw.tolist(),
                        norm_eps=1e-5, **v)
    assert np.array_equal(r["xq"], np.array(ref["xq"], np.uint8))
    np.testing.assert_allclose(r["s_x"], ref["s_x"], rtol=1e-15)
    assert np.array_equal(r["aq_shared"], np.array(ref["aq_shared"], np.uint8))
    assert np.array_equal(r["aq_routed"], np.array(ref["aq_routed"], np.uint8))
    np.testing.assert_allclose(r["ref"], np.array(ref["ref"]), rtol=1e-12, atol=1e-300)
    # the norm changes the step (the weights are not all one and rows are not unit RMS)
    assert not np.array_equal(r["xq"], ffn.forward(x, lg, experts, E, **v)["xq"])
