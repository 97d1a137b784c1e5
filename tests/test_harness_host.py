"""Host checks of the parity harness's own helpers (no GPU): the reference a token's
output is compared with when its re-quantised codes differ from the oracle's, and the
count of routed experts streamed by a batch above one launch."""

import numpy as np

import workloads as W
from harness import chunked_active, conditioned_ref, ordv
from oracle import ffn
from oracle import fp8 as ofp8


def _problem(seed=3, M=6, K=256, I=256, E=3):
    x = W.activations(seed, M, K, "cpu")
    lg = W.router_logits(seed, M, E, "cpu")
    ws = [W.expert(seed, s, K, I, "cpu").numpy() for s in range(E + 1)]
    return ffn.forward(W.bits(x), W.bits(lg), ws, E), ws


def test_conditioned_ref_of_the_oracles_own_codes_is_the_oracle():
    ref, ws = _problem()
    rows = np.arange(ref["ref"].shape[0])
    got = conditioned_ref(ref, ref, lambda s: ws[s], 3, rows)
    assert np.array_equal(got, ref["ref"])
    dense, wd = _problem(E=0)
    assert np.array_equal(conditioned_ref(dense, dense, lambda s: wd[s], 0, rows), dense["ref"])


def test_conditioned_ref_follows_a_flipped_code():
    """One intermediate code moved by one step changes exactly that token's reference,
    by that step times the code's row of W2 (and the gate, for a routed row)."""
    ref, ws = _problem()
    E, m, j = 3, 2, 5
    for kind in ("shared", "routed"):
        gpu = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in ref.items()}
        c = int(gpu["aq_" + kind][m, j])
        assert c & 0x7F not in (0, 0x7E)
        gpu["aq_" + kind][m, j] = c + 1  # one step away from zero
        assert np.abs(ordv(gpu["aq_" + kind]) - ordv(ref["aq_" + kind])).sum() == 1
        rows = np.arange(ref["ref"].shape[0])
        got = conditioned_ref(gpu, ref, lambda s: ws[s], E, rows)
        step = (ofp8.e4m3_decode(np.array([c + 1], np.uint8)) - ofp8.e4m3_decode(np.array([c], np.uint8)))[0]
        slot = E if kind == "shared" else int(ref["expert"][m])
        w = ws[slot]
        g = 1.0 if kind == "shared" else ref["gate"][m]
        want = g * step * ref["s_a_" + kind][m] * ofp8.e4m3_decode(w.w2[j]) * w.s2
        assert np.allclose(got[m] - ref["ref"][m], want, rtol=1e-9, atol=1e-12 * np.abs(ref["ref"]).max())
        others = np.arange(ref["ref"].shape[0]) != m
        assert np.array_equal(got[others], ref["ref"][others])


def test_chunked_active_counts_runs_of_the_expert_order():
    assert chunked_active([0, 1] * 20) == 1 + 2 + 1  # sorted: 20 zeros then 20 ones
    assert chunked_active([3, 1, 3, 2]) == 3          # one launch: its distinct experts
    assert chunked_active([5] * 17) == 2              # one expert over two launches
    assert chunked_active(list(range(40))) == 40


def test_smoke_calls_the_harness_with_its_current_signature():
    """smoke() runs only on a GPU; check here that its calls into the harness bind."""
    import ast
    import inspect
    import os

    import harness

    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "__graft_entry__.py")).read()
    calls = [n for n in ast.walk(ast.parse(src)) if isinstance(n, ast.Call)
             and isinstance(n.func, ast.Name) and n.func.id in ("check_all", "Problem")]
    assert calls
    for call in calls:
        sig = inspect.signature(getattr(harness, call.func.id))
        sig.bind(*[None] * len(call.args), **{k.arg: None for k in call.keywords})


def test_binding_structures_construct():
    """The binding's host structures build as the harness and smoke() use them."""
    import dataclasses

    import fp8_moe_ffn_amd as F

    v = F.Variant(1, 0.5, 0.25)
    assert (v.gate_on_input, v.x_scale, v.a_scale) == (1, 0.5, 0.25)
    assert dataclasses.is_dataclass(F.DebugOut)
    names = [f.name for f in dataclasses.fields(F.DebugOut)]
    assert names == [n for n, _ in F.DebugPtrs._fields_]


def test_conditioned_step_of_the_oracles_own_codes_is_the_oracle():
    """The stage-wise reference from the oracle's own activation codes reproduces the
    oracle (output gate, input gate, static intermediate scale)."""
    from harness import conditioned_step
    for kw in (dict(), dict(gate_on_input=True), dict(a_scale=0.01)):
        seed, M, K, I, E = 3, 6, 256, 256, 3
        x = W.activations(seed, M, K, "cpu")
        lg = W.router_logits(seed, M, E, "cpu")
        ws = [W.expert(seed, s, K, I, "cpu").numpy() for s in range(E + 1)]
        ref = ffn.forward(W.bits(x), W.bits(lg), ws, E, **kw)
        rows = np.arange(M)
        c = conditioned_step(ref, ref, lambda s: ws[s], E, rows, kw.get("gate_on_input", False),
                             kw.get("a_scale"))
        for k in ("aq_shared", "s_a_shared", "aq_routed", "s_a_routed", "ref"):
            assert np.array_equal(c[k], ref[k]), (kw, k)


def _as_gpu(ref, E):
    """The oracle's result in the form run_gpu returns (float32 scales, bf16 output bits)."""
    from harness import streamed_active
    g = {k: np.array(ref[k]) for k in ("xq", "aq_shared", "aq_routed", "out")}
    for k in ("s_x", "gate", "s_a_shared", "s_a_routed"):
        g[k] = np.asarray(ref[k], np.float64).astype(np.float32)
    g["expert"] = np.asarray(ref["expert"], np.int32)
    g["num_active"] = np.array([streamed_active(ref["expert"]) if E else 0], np.int32)
    return g


def test_check_all_is_strict_where_the_path_is_exact():
    """The parity checks reject what they must: one activation code one step off, a scale
    one float32 step off, and a token whose output misses the bar although its codes equal
    the oracle's (mistakes planted in a copy of the oracle's own result, which itself
    passes with no token conditioned)."""
    import pytest

    from harness import check_all
    ref, ws = _problem(M=6, I=1024, E=3)
    weights = lambda s: ws[s]
    s = check_all(_as_gpu(ref, 3), ref, 3, weights, max_conditioned=0)
    assert s["tokens_conditioned"] == 0 and s["tokens_x_conditioned"] == 0 and s["tokens_codes_differ"] == 0
    g = _as_gpu(ref, 3)
    c = int(g["xq"][1, 7])
    g["xq"][1, 7] = c + 1 if (c & 0x7F) < 0x7E else c - 1
    with pytest.raises(AssertionError, match="xq differs"):
        check_all(g, ref, 3, weights)
    g = _as_gpu(ref, 3)
    g["s_x"][2] = np.nextafter(g["s_x"][2], np.float32(1))
    with pytest.raises(AssertionError, match="s_x differs"):
        check_all(g, ref, 3, weights)
    g = _as_gpu(ref, 3)
    g["out"][4] = ofp8.f64_to_bf16(ofp8.bf16_to_f64(g["out"][4]) * 1.05)
    with pytest.raises(AssertionError, match="miss the output bar"):
        check_all(g, ref, 3, weights)
